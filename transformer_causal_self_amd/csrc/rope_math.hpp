// rope_math.hpp -- the rotation of one RoPE channel pair, shared by every
// kernel that rotates (the RoPE pass, the decode-step preparation and the
// prefill kernel's query load), so they all produce the same bits.
//
// A pair (x1, x2) turns by the angle whose float32 cosine and sine are
// (c, s): [[c, -s], [s, c]] ("Transformer" (ai-notes) -- RoPE; "The
// Transformer architecture" -- Now: RoPE).  Written with explicit fused
// multiply-adds so that no kernel's compiler contracts it differently.
#pragma once

namespace rocattn {

__device__ inline void rope_turn(float x1, float x2, float c, float s, float& y1, float& y2) {
    y1 = fmaf(x1, c, -(x2 * s));
    y2 = fmaf(x1, s, x2 * c);
}

}  // namespace rocattn
