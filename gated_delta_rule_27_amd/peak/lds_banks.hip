// lds_banks.hip — which lanes of a wave share an LDS clock on this device, for
// each access width, measured with the SQ_LDS_BANK_CONFLICT counter (run under
// rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_LDS_IDX_ACTIVE).  Not
// part of the linear-attention library; the layouts of the chunk kernels' LDS
// tiles follow from what it shows.
//
// Dispatch order: for each access kind (ds_read_b128, ds_read_b64,
// ds_write_b64, ds_write_b128) and each partner lane b = 1..63, one launch in
// which only lanes 0 and b are active, lane 0 at byte 0 and lane b at byte
// 256 (the same bank if there are 64 four-byte banks): a conflict is counted
// exactly when lane b is served in the same clock as lane 0.  Then lane 1 at
// byte offsets 16 .. 512 for the two read kinds (the bank count).  Then the
// same partner-lane sweep for the 2- and 4-byte kinds (ds_read_u16,
// ds_read_b32, ds_write_b16, ds_write_b32), and lane 1 at byte offsets 2
// (the same dword), 4, 64, 128 and 256 for each of them (offsets rounded down
// to 4 bytes for the 4-byte kinds).  Last, ds_read2_b64 with its second
// address 32 bytes above the first (the form the compiler makes of two 8-byte
// reads from one base): the partner-lane sweep, then lane 1 at byte offsets
// 8 .. 256.  Every address stays below 16 KiB of the workgroup's LDS.
#include <hip/hip_runtime.h>
#include <cstdio>

typedef __attribute__((__vector_size__(16))) int i4;
typedef __attribute__((__vector_size__(8))) int i2;

namespace {

constexpr int kBytes = 16 * 1024;
constexpr int kIters = 4096;

template <int KIND>
__global__ __launch_bounds__(64) void lane_pair(int* out, int b, int off)
{
    __shared__ __align__(16) char lds[kBytes];
    const int l = threadIdx.x;
    for (int i = l; i < kBytes / 4; i += 64) reinterpret_cast<int*>(lds)[i] = i;
    __syncthreads();
    int acc = 0;
    if (l == 0 || l == b) {
        const unsigned a0 = (unsigned)(uintptr_t)lds + (l == 0 ? 0 : off);
        for (int it = 0; it < kIters; ++it) {
            // two accesses per round, waited for inside the same asm block
            if (KIND == 0) {
                i4 v0, v1;
                asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(v0), "=v"(v1) : "v"(a0));
                acc += v0[0] ^ v1[3];
            } else if (KIND == 1) {
                i2 v0, v1;
                asm volatile("ds_read_b64 %0, %2\n\tds_read_b64 %1, %2\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(v0), "=v"(v1) : "v"(a0));
                acc += v0[0] ^ v1[1];
            } else if (KIND == 2) {
                const i2 w = {it, l};
                asm volatile("ds_write_b64 %0, %1\n\tds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                             :: "v"(a0), "v"(w) : "memory");
            } else if (KIND == 3) {
                const i4 w = {it, l, acc, 3};
                asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                             :: "v"(a0), "v"(w) : "memory");
            } else if (KIND == 4) {
                int v0, v1;
                asm volatile("ds_read_u16 %0, %2\n\tds_read_u16 %1, %2\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(v0), "=v"(v1) : "v"(a0));
                acc += v0 ^ v1;
            } else if (KIND == 5) {
                int v0, v1;
                asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %2\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(v0), "=v"(v1) : "v"(a0));
                acc += v0 ^ v1;
            } else if (KIND == 6) {
                const int w = it + l;
                asm volatile("ds_write_b16 %0, %1\n\tds_write_b16 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                             :: "v"(a0), "v"(w) : "memory");
            } else if (KIND == 7) {
                const int w = it + l;
                asm volatile("ds_write_b32 %0, %1\n\tds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                             :: "v"(a0), "v"(w) : "memory");
            } else {
                i4 v0, v1;
                asm volatile("ds_read2_b64 %0, %2 offset1:4\n\tds_read2_b64 %1, %2 offset1:4\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(v0), "=v"(v1) : "v"(a0));
                acc += v0[0] ^ v1[3];
            }
        }
    }
    __syncthreads();
    out[blockIdx.x * 64 + l] = acc + reinterpret_cast<int*>(lds)[l];
}

}  // namespace

int main()
{
    int* d = nullptr;
    if (hipMalloc(&d, 64 * 64 * sizeof(int)) != hipSuccess) return 1;
    const char* kinds[] = {"ds_read_b128", "ds_read_b64", "ds_write_b64", "ds_write_b128"};
    for (int kind = 0; kind < 4; ++kind) {
        for (int b = 1; b < 64; ++b) {
            if (kind == 0) hipLaunchKernelGGL(lane_pair<0>, dim3(64), dim3(64), 0, 0, d, b, 256);
            if (kind == 1) hipLaunchKernelGGL(lane_pair<1>, dim3(64), dim3(64), 0, 0, d, b, 256);
            if (kind == 2) hipLaunchKernelGGL(lane_pair<2>, dim3(64), dim3(64), 0, 0, d, b, 256);
            if (kind == 3) hipLaunchKernelGGL(lane_pair<3>, dim3(64), dim3(64), 0, 0, d, b, 256);
        }
        printf("%s: partner lanes 1..63 launched\n", kinds[kind]);
    }
    const int offs[] = {16, 32, 64, 128, 256, 512};
    for (int o : offs) hipLaunchKernelGGL(lane_pair<0>, dim3(64), dim3(64), 0, 0, d, 1, o);
    for (int o : offs) hipLaunchKernelGGL(lane_pair<1>, dim3(64), dim3(64), 0, 0, d, 1, o);
    printf("bank-width launches done\n");
    const char* skinds[] = {"ds_read_u16", "ds_read_b32", "ds_write_b16", "ds_write_b32"};
    for (int kind = 4; kind < 8; ++kind) {
        for (int b = 1; b < 64; ++b) {
            if (kind == 4) hipLaunchKernelGGL(lane_pair<4>, dim3(64), dim3(64), 0, 0, d, b, 256);
            if (kind == 5) hipLaunchKernelGGL(lane_pair<5>, dim3(64), dim3(64), 0, 0, d, b, 256);
            if (kind == 6) hipLaunchKernelGGL(lane_pair<6>, dim3(64), dim3(64), 0, 0, d, b, 256);
            if (kind == 7) hipLaunchKernelGGL(lane_pair<7>, dim3(64), dim3(64), 0, 0, d, b, 256);
        }
        printf("%s: partner lanes 1..63 launched\n", skinds[kind - 4]);
    }
    const int soffs[] = {2, 4, 64, 128, 256};
    for (int o : soffs) hipLaunchKernelGGL(lane_pair<4>, dim3(64), dim3(64), 0, 0, d, 1, o);
    for (int o : soffs) hipLaunchKernelGGL(lane_pair<5>, dim3(64), dim3(64), 0, 0, d, 1, o & ~3);
    for (int o : soffs) hipLaunchKernelGGL(lane_pair<6>, dim3(64), dim3(64), 0, 0, d, 1, o);
    for (int o : soffs) hipLaunchKernelGGL(lane_pair<7>, dim3(64), dim3(64), 0, 0, d, 1, o & ~3);
    printf("2- and 4-byte launches done\n");
    for (int b = 1; b < 64; ++b) hipLaunchKernelGGL(lane_pair<8>, dim3(64), dim3(64), 0, 0, d, b, 256);
    const int r2offs[] = {8, 16, 32, 64, 128, 160, 256};
    for (int o : r2offs) hipLaunchKernelGGL(lane_pair<8>, dim3(64), dim3(64), 0, 0, d, 1, o);
    if (hipDeviceSynchronize() != hipSuccess) return 2;
    printf("ds_read2_b64 launches done\n");
    return hipFree(d) == hipSuccess ? 0 : 3;
}
