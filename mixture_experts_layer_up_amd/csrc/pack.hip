// pack.hip -- one-time relayout of expert weights into MFMA fragments.
//
// A [K, N] weight (N contiguous) is rewritten so that the B operand of one
// 16x16x32 bf16 MFMA -- 32 K rows by 16 columns, lane l holding the 8
// consecutive K values of column l % 16 starting at row 8 (l / 16) -- is
// one contiguous 1 KiB block, and so that everything one GEMM block streams
// (one 64-column slab of one expert: 4 column tiles over all of K) is one
// contiguous region, chunk after chunk:
//   packed[(((e * n_slabs + slab) * KC + kc) * 4 + t) * 512 + 8 l + i]
//     = W[e][32 kc + 8 (l / 16) + i][col(4 slab + t) + l % 16]
// The grouped GEMMs then stream each slab with fully coalesced 16-byte loads
// straight into registers, as one sequential read.
//
// For w13 the 16-column tiles alternate gate and up tiles of the same
// columns (tile 2j = gate columns [16j, 16j+16), tile 2j+1 = the matching up
// columns at I + 16j), so one block of the gate_up GEMM owns matching gate
// and up outputs and can apply SwiGLU in its epilogue.
#include "device_common.h"
#include "kernels.h"

namespace moe_lora {
namespace {

__global__ __launch_bounds__(256) void pack_kernel(PackArgs a)
{
    const size_t f = (size_t)blockIdx.x * 256 + threadIdx.x;  // one 16-byte lane fragment
    const int KC = a.K >> 5;
    const int NT = a.N >> 4;
    const size_t total = (size_t)a.E_l * NT * KC * kWave;
    if (f >= total)
        return;
    const int lane = (int)(f & (kWave - 1));
    size_t rest = f >> 6;
    const int t = (int)(rest & 3);  // tile inside the 4-tile slab
    rest >>= 2;
    const int kc = (int)(rest % KC);
    rest /= KC;
    const int n_slabs = NT >> 2;
    const int slab = (int)(rest % n_slabs);
    const int e = (int)(rest / n_slabs);
    const int nt = slab * 4 + t;
    const int col = a.I > 0 ? (nt & 1) * a.I + (nt >> 1) * 16 + (lane & 15)
                            : nt * 16 + (lane & 15);
    const int k0 = kc * 32 + (lane >> 4) * 8;
    const uint16_t *src = a.src + ((size_t)e * a.K + k0) * a.N + col;
    u32x4 v;
    v.x = (uint32_t)src[0] | ((uint32_t)src[(size_t)1 * a.N] << 16);
    v.y = (uint32_t)src[(size_t)2 * a.N] | ((uint32_t)src[(size_t)3 * a.N] << 16);
    v.z = (uint32_t)src[(size_t)4 * a.N] | ((uint32_t)src[(size_t)5 * a.N] << 16);
    v.w = (uint32_t)src[(size_t)6 * a.N] | ((uint32_t)src[(size_t)7 * a.N] << 16);
    store16(a.dst + f * 8, v);
}

// One-time relayout of LoRA A stacks (the shrink's operand) into 64-value K
// chunks that hold all rank rows of the chunk contiguously (kernels.h,
// lora_a_chunks).  The shrink kernels read a stack chunk by chunk, every rank
// row at once; row-major stacks spread each chunk over r rows 2K bytes
// apart.  One thread per 16-byte output piece; K % 32 == 0, so a piece lies
// wholly inside K or wholly in the zero padding.
__global__ __launch_bounds__(256) void pack_lora_a_kernel(PackAArgs a)
{
    const size_t f = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int C = lora_a_chunks(a.K);
    const size_t total = (size_t)a.stacks * C * a.r * 8;
    if (f >= total)
        return;
    const int u = (int)(f & 7);  // 16-byte piece inside the 64-value row chunk
    size_t rest = f >> 3;
    const int q = (int)(rest % a.r);
    rest /= a.r;
    const int c = (int)(rest % C);
    const size_t stack = rest / C;
    const int k0 = c * 64 + u * 8;
    u32x4 v{0u, 0u, 0u, 0u};
    if (k0 < a.K)
        v = load16(a.src + (stack * a.r + q) * a.K + k0);
    store16(a.dst + f * 8, v);
}

} // namespace

hipError_t launch_pack_lora_a(const PackAArgs &a, hipStream_t s)
{
    const size_t total = (size_t)a.stacks * lora_a_chunks(a.K) * a.r * 8;
    if (total == 0)
        return hipSuccess;
    const size_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(pack_lora_a_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pack(const PackArgs &a, hipStream_t s)
{
    const size_t total = (size_t)a.E_l * (a.N >> 4) * (a.K >> 5) * kWave;
    if (total == 0)
        return hipSuccess;
    const size_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_lora
