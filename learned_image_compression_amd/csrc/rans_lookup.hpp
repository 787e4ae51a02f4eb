// rans_lookup.hpp -- the decoders' symbol lookup (the lane and the
// interleaved decoder share the decoder table set, so they share this step).
// Inverse-CDF decoding keyed by the low state bits (torch_ans "Usage"): a
// per-row table of 2^q buckets gives the slot holding each bucket's lowest
// cumulative value, and one 8-byte read of start - 1 for the next four slots
// settles most steps.
#pragma once

#include "rans_internal.hpp"

namespace rans {

// Decoder tables: [meta | cdfm1 | first], in LDS from address 0 or in the
// workspace.  cdfm1[k] = start(k) - 1 mod 2^16 (the terminal 65536 becomes
// 65535), so cum >= start(k) is cum > cdfm1[k] and f(k) = cdfm1[k+1] -
// cdfm1[k] mod 2^16.
struct DecTables {
    uint32_t q;              // 2^q buckets per row
    uint32_t shift;          // 16 - q: cumulative value -> bucket
    uint32_t K;
};

// The common-case arithmetic of one step.  The bucket's first slot fs and the
// four entries cdfm1[fs .. fs+3] (one 8-byte read) resolve any cum that falls
// in slots fs .. fs+2.  Entries increase along a valid row and its terminal
// entry is 65535, so a comparison with a later entry can only hold when the
// earlier ones do, except past the terminal, where the slot it gives is at
// least the escape slot and so never taken for an ordinary one.
struct Lookup {
    uint32_t bucket, slot, f, rr;
    bool beyond;
    uint64_t xn;   // the state after the step, before renormalisation
};

template <class Tab>
__device__ __forceinline__ Lookup lookup_step(const RowMeta &m, uint64_t x, const DecTables &t,
                                              const Tab &tab)
{
    Lookup s;
    const uint32_t xlo = (uint32_t)x, xhi = (uint32_t)(x >> 32);
    const uint32_t cum = xlo & (kTotal - 1);
    s.bucket = cum >> t.shift;
    const uint32_t fs = tab.template load<uint16_t>(m.lut + 2 * s.bucket);
    const uint64_t v = tab.u16x4(m.base + 2 * fs);
    const uint32_t wlo = (uint32_t)v, whi = (uint32_t)(v >> 32);   // cdfm1[fs..fs+1], [fs+2..fs+3]
    const bool c1 = cum > (wlo >> 16);
    const bool c2 = cum > (whi & 0xFFFFu);
    s.beyond = cum > (whi >> 16);
    s.slot = fs + (c1 ? 1u : 0u) + (c2 ? 1u : 0u);
    // the slot's cdfm1 pair (start - 1, next start - 1) as one packed word;
    // f = its high half minus its low half and rr = cum - start, both mod
    // 2^16 (16-bit subtractions on the halves, upper bits cleared)
    const uint32_t pair = c2 ? whi : (c1 ? __builtin_amdgcn_alignbit(whi, wlo, 16) : wlo);
    const uint32_t xlo_m1 = xlo - 1u;   // cum - 1 mod 2^16 in the low half
    asm("v_sub_u16_sdwa %0, %1, %1 dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:WORD_0"
        : "=v"(s.f) : "v"(pair));
    asm("v_sub_u16_sdwa %0, %1, %2 dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:WORD_0"
        : "=v"(s.rr) : "v"(xlo_m1), "v"(pair));
    // f * (x >> 16) + rr with x >> 16 < 2^48 split at bit 32
    const uint32_t mid = __builtin_amdgcn_alignbit(xhi, xlo, 16);
    const uint64_t lo64 = (uint64_t)s.f * mid + s.rr;
    const uint32_t nhi = (uint32_t)(lo64 >> 32) + __umul24(s.f, xhi >> 16);
    s.xn = ((uint64_t)nhi << 32) | (uint32_t)lo64;
    return s;
}

}  // namespace rans
