// Cross-lane combines on VALU permutes instead of LDS-routed shuffles.
//
// v_permlane16_swap / v_permlane32_swap (gfx950) swap rows of 16 lanes
// (halves of 32) between two registers; called with the same value twice they
// hand every lane both values of its pair (lane l and l ^ 16, or l ^ 32), so
// op(a, b) equals a shuffle by xor 16 (32) followed by op, bit for bit, for a
// commutative op. Inside a row of 16 lanes, DPP quad permutations and the
// half-row / row mirrors pair every lane with one in the other quad / half,
// which joins the row for max and sum (the sum's association differs from an
// xor butterfly's). Every lane of the combined group must be active.
#pragma once

namespace nosa {

__device__ inline float pl_bits(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ inline unsigned pl_u(float f) { return __builtin_bit_cast(unsigned, f); }

__device__ inline float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(pl_u(v), pl_u(v), false, false);
  return fmaxf(pl_bits(r[0]), pl_bits(r[1]));
}
__device__ inline float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(pl_u(v), pl_u(v), false, false);
  return pl_bits(r[0]) + pl_bits(r[1]);
}
__device__ inline float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(pl_u(v), pl_u(v), false, false);
  return fmaxf(pl_bits(r[0]), pl_bits(r[1]));
}
__device__ inline float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(pl_u(v), pl_u(v), false, false);
  return pl_bits(r[0]) + pl_bits(r[1]);
}

template <int CTRL>
__device__ inline float dpp_f32(float v) {
  return pl_bits(static_cast<unsigned>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(pl_u(v)), CTRL, 0xF, 0xF, true)));
}
// v of lane l + K (K > 0) or l - |K| (K < 0) in the same row of 16 lanes;
// a lane whose source falls outside its row keeps its own v (as __shfl_down
// / __shfl_up with width 16)
template <int K>
__device__ inline float row_shift(float v) {
  constexpr int ctrl = K > 0 ? 0x100 + K : 0x110 - K;   // row_shl:K / row_shr:-K
  return pl_bits(static_cast<unsigned>(__builtin_amdgcn_update_dpp(
      static_cast<int>(pl_u(v)), static_cast<int>(pl_u(v)), ctrl, 0xF, 0xF, false)));
}

// max / sum over each row of 16 lanes, left in every lane of the row
__device__ inline float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));     // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));     // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));    // row_half_mirror
  return fmaxf(v, dpp_f32<0x140>(v)); // row_mirror
}
__device__ inline float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  return v + dpp_f32<0x140>(v);
}

}  // namespace nosa
