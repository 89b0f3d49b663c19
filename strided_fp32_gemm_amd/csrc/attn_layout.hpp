// attn_layout.hpp -- LDS layout of the fused attention kernel's key blocks.
//
// Plain constexpr arithmetic (no HIP headers), shared by the kernel and the
// host-side checker, so the layout the checker proves free of bank conflicts
// is the one the kernel uses.
//
// A buffer holds one 64-key block: K rows of kAttnKPitch floats, then V rows
// of kAttnVPitch floats.  Staging slot s (0 .. 1023) is key row s / 16, head
// dimensions 4*(s % 16) .. +3 (one 16-byte global load and LDS write).  The
// 16-byte chunk c of K row `key` sits at chunk c ^ attn_k_flip(key): rows
// whose key bits 2 and 3 differ swap chunks in pairs (c and c ^ 4), which
// keeps the fragment reads below conflict-free at a pitch of 68 floats.
//
// Fragment reads of lane l (lq = l % 16, lh = l / 16) in 16 bytes:
//  - K: key 16*kb + lq, head dimensions 16*lh + 4*j .. +3 (score step group j);
//  - V: key 16*kb + 4*lh + r, head dimensions 4*lq .. +3 (the four P V
//    products of one step take head dimensions 4*i + nb for their rows i).
#pragma once

namespace sgemm {

constexpr int kAttnD = 64;                                    // head dimension
constexpr int kAttnBlockKeys = 64;                            // keys per LDS block
constexpr int kAttnKPitch = kAttnD + 4;                       // K row pitch (floats)
constexpr int kAttnVPitch = kAttnD;                           // V row pitch (floats)
constexpr int kAttnKFloats = kAttnBlockKeys * kAttnKPitch;    // K part of a buffer
constexpr int kAttnBufFloats = kAttnKFloats + kAttnBlockKeys * kAttnVPitch;
constexpr int kAttnSlots = kAttnBlockKeys * kAttnD / 4;       // 16-byte slots per K (or V) block

constexpr int attn_k_flip(int key) { return (((key >> 2) ^ (key >> 3)) & 1) << 2; }

// Float offsets inside a buffer.
constexpr int attn_k_slot(int s) {
    return (s >> 4) * kAttnKPitch + 4 * ((s & 15) ^ attn_k_flip(s >> 4));
}
constexpr int attn_v_slot(int s) { return kAttnKFloats + (s >> 4) * kAttnVPitch + 4 * (s & 15); }
constexpr int attn_k_frag(int lane, int kb, int j) {
    return (16 * kb + (lane & 15)) * kAttnKPitch + 4 * ((4 * (lane >> 4) + j) ^ attn_k_flip(16 * kb + (lane & 15)));
}
constexpr int attn_v_frag(int lane, int kb, int r) {
    return kAttnKFloats + (16 * kb + 4 * (lane >> 4) + r) * kAttnVPitch + 4 * (lane & 15);
}

}  // namespace sgemm
