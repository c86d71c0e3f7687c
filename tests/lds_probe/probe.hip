// LDS read-pattern probe: each dispatch runs one wave that issues 8 reads per
// iteration at per-lane offsets from a table (b128 row reads or b64
// transposing reads), so SQ_LDS_BANK_CONFLICT per dispatch measures one
// pattern.  Offsets are checked on the host: < 65536 - 16, aligned.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <int KIND>
__global__ __launch_bounds__(64) void probe(const int* __restrict__ offs, int iters, int* __restrict__ out) {
    __shared__ __attribute__((aligned(1024))) char lds[65536];
    const int lane = threadIdx.x;
    for (int i = lane; i < 65536 / 4; i += 64) reinterpret_cast<int*>(lds)[i] = i;
    __syncthreads();
    int o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = offs[j * 64 + lane];
    int acc = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (KIND == 0) {
                const i32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(
                    (__attribute__((address_space(3))) char*)lds + o[j]);
                acc += v[0] ^ v[3];
            } else {
                const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    reinterpret_cast<__attribute__((address_space(3))) i16x4*>((__attribute__((address_space(3))) char*)lds + o[j]));
                acc += v[0] ^ v[3];
            }
        }
        asm volatile("" ::: "memory");
    }
    out[lane] = acc;
}
int main(int argc, char** argv) {
    FILE* f = fopen(argv[1], "r");
    if (!f) return 2;
    int n;
    if (fscanf(f, "%d", &n) != 1) return 3;
    std::vector<int> kinds(n), offs(size_t(n) * 512);
    for (int t = 0; t < n; ++t) {
        if (fscanf(f, "%d", &kinds[t]) != 1) return 4;
        for (int k = 0; k < 512; ++k) {
            if (fscanf(f, "%d", &offs[size_t(t) * 512 + k]) != 1) return 5;
            const int a = offs[size_t(t) * 512 + k];
            if (a < 0 || a > 65536 - 16 || a % (kinds[t] == 0 ? 16 : 8) != 0) { printf("bad offset %d test %d\n", a, t); return 6; }
        }
    }
    fclose(f);
    int *d_offs, *d_out;
    if (hipMalloc(&d_offs, offs.size() * 4) != hipSuccess || hipMalloc(&d_out, 64 * 4) != hipSuccess) return 7;
    if (hipMemcpy(d_offs, offs.data(), offs.size() * 4, hipMemcpyHostToDevice) != hipSuccess) return 8;
    for (int t = 0; t < n; ++t) {
        if (kinds[t] == 0)
            probe<0><<<1, 64>>>(d_offs + size_t(t) * 512, 16, d_out);
        else
            probe<1><<<1, 64>>>(d_offs + size_t(t) * 512, 16, d_out);
        if (hipDeviceSynchronize() != hipSuccess) { printf("launch failed at %d\n", t); return 9; }
    }
    printf("ran %d tests\n", n);
    return 0;
}
