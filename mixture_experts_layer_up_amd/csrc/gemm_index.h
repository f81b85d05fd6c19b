// gemm_index.h -- where the decode-shaped GEMM's B-operand loads read.
//
// The decode GEMM (expert_gemm.hip) gives each of its 4 waves a sequence of
// virtual K chunks: first its main chunks (chunks w, w + 4, ... of the
// packed weight slab, K / 32 in all), then its LoRA expand chunks (32 rank
// positions of the concatenated adapters' B columns each).  Every lane loads
// 16 bytes per B tile per chunk, and a rank that is not a multiple of 8 adds
// 2-byte loads of the expand row.  Every load is issued whatever the chunk
// kind, so that all paths have the same loads in flight; the address of a
// load whose value is not used must still be a valid one.
//
// This header is the single definition of those addresses.  It holds plain
// integer arithmetic only, so a host program can run it over every (wave,
// chunk, lane, tile) of a shape and check that each address lies inside its
// buffer: the host-side bounds test does exactly that.
#pragma once

#include <stddef.h>

#if defined(__HIP__)
#define MOE_LORA_HD __host__ __device__
#else
#define MOE_LORA_HD
#endif

namespace moe_lora {

// Per-launch constants of the decode GEMM's B loads.
struct DecodeBShape {
    int KC;         // main K chunks: K / 32
    int NS;         // 16-column tiles per work item (4: one 64-column slab)
    int n_slabs;    // 64-column slabs per expert
    int gated;      // 1: gate_up (gate and up tiles alternate), 0: down
    int I;          // inter (the gate_up column map)
    int L, r, rp;   // adapters, LoRA rank, rank rounded up to 8
    int E_l;        // local experts
    int n_canon;    // output columns of the unpacked weight (2I or H)
    int lb_shared;  // the LoRA B stack holds one set per adapter
};

// Main chunks of a wave: chunks wave, wave + 4, ... below KC.
MOE_LORA_HD inline int decode_main_chunks(int KC, int wave)
{
    return wave < KC ? (KC - wave + 3) >> 2 : 0;
}

// The loads one lane issues for B tile n of its virtual chunk vc.
struct DecodeBLoad {
    int from_lora;    // the 16-byte load reads the LoRA B stack (1) or the packed weights (0)
    size_t off16;     // element offset of the 16-byte load in that buffer
    size_t lora_row;  // element offset of the lane's LoRA B row (its stack and output column)
    int q0;           // first of the lane's 8 rank positions in that row
    int aid;          // adapter of the expand chunk (L or more: past the last adapter)
};

// vc: the wave's virtual chunk; nm: its main chunks; le, slab: the work
// item's local expert and 64-column slab; n: B tile (0 .. NS - 1).
//  * A main chunk (vc < nm) reads fragment (chunk wave + 4 vc, tile n) of
//    the item's packed slab.
//  * An expand chunk covers rank positions g .. g + 7 of the concatenated
//    adapters, g = 32 (expand chunk index) + 8 (lane / 16): adapter g / rp,
//    position g % rp.  Its row is that adapter's B column of the lane's
//    output column (the last adapter's when g runs past the last one: those
//    K positions meet zero activations).  With r % 8 == 0 the 16-byte load
//    reads the row at q0; otherwise it reads the item's first weight
//    fragment (valid, unused) and the 2-byte loads read positions
//    min(q0 + i, r - 1), i < 8.
MOE_LORA_HD inline DecodeBLoad decode_b_load(const DecodeBShape &s, int wave, int lane, int vc,
                                             int nm, int le, int slab, int n)
{
    DecodeBLoad d;
    const bool main = vc < nm;
    const size_t slab_base =
        ((size_t)le * s.n_slabs + slab) * (size_t)s.KC * s.NS * 512 + (size_t)lane * 8;
    const int kc = wave + 4 * (main ? vc : 0);
    const size_t frag = slab_base + ((size_t)kc * s.NS + n) * 512;
    const int g = ((vc - nm) * 4 + wave) * 32 + (lane >> 4) * 8;
    const int aid = main ? 0 : g / s.rp;
    d.aid = aid;
    d.q0 = main ? 0 : g - aid * s.rp;
    const int aid_c = aid < s.L - 1 ? aid : (s.L > 0 ? s.L - 1 : 0);
    const int col = s.gated ? (n & 1) * s.I + (slab * 2 + (n >> 1)) * 16 + (lane & 15)
                            : (slab * s.NS + n) * 16 + (lane & 15);
    const size_t stack = s.lb_shared ? (size_t)aid_c : (size_t)aid_c * s.E_l + le;
    d.lora_row = (stack * s.n_canon + col) * (size_t)s.r;
    const bool rank8 = (s.r & 7) == 0;
    d.from_lora = (!main && rank8) ? 1 : 0;
    // a main chunk's fragment; an expand chunk's row (rank % 8 == 0), else
    // the item's first fragment, which exists whether or not this wave has
    // main chunks (a wave past K / 32 has none)
    d.off16 = main ? frag : rank8 ? d.lora_row + d.q0 : slab_base;
    return d;
}

} // namespace moe_lora
