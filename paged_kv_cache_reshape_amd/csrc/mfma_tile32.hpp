// Matrix-core attention for 32 query rows per wave on 32x32x16 bfloat16
// tiles (v_mfma_f32_32x32x16_bf16), used by the prefill kernel and by the
// decode of 32 query heads per kv head over 32-token blocks.
//
// On MI355X this instruction sustains about twice the rate per flop of the
// 16x16x32 form (measured: 2.3 against 1.3 PFLOP/s with independent
// accumulators), and prefill -- many query rows against the same keys -- has
// the rows to fill it.  What is computed is the online softmax of the pages
// (LLAISYS README, self-attention item; barellm README, paged-cache list),
// for one 32-key fold at a time:
//
//   * S^T = K q^T: A = 32 K rows (lane l: token l % 32, d = 16 i + 8 (l / 32)
//     .. + 7), B = the 32 query rows held in registers (lane l: row l % 32,
//     same d).  The result lane l holds query row l % 32 against tokens
//     row32(l, r) = 8 (r / 4) + 4 (l / 32) + r % 4, r < 16, so each lane sees
//     one row: its running maximum needs only the other half of the wave
//     (lane l ^ 32);
//   * scores past a row's position are masked (only in folds where a key can
//     lie past some row), and the scale enters the exponent,
//     p = exp2(c s - m) with c > 0, against a lazily kept maximum that moves
//     only when a score passes it by more than 8 (base 2);
//   * O += P V: registers 8 h .. 8 h + 7 of the scores are already the A
//     operand of the h-th 16-key product (lane l: row l % 32, keys
//     16 h + 8 (s / 4) + 4 (l / 32) + s % 4 for slot s).  The B operand takes
//     the same keys of V: two ds_read_b64_tr_b16 of four tokens each, rows
//     16 h + 4 (l / 32) and 16 h + 8 + 4 (l / 32);
//   * weights are split hi + lo (hi = p with its low 16 bits cleared, lo =
//     bf16(p - hi)), two products, so they keep 16 significant bits.
#pragma once

#include "mfma_attn.hpp"

namespace pa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int D>
struct Tile32Shape {
  static constexpr int DK = D / 16;  // 16-wide d slices of q.k
  static constexpr int DT = D / 32;  // 32-wide d tiles of the output
  // LDS row pitches, bytes.  K rows are read 16 bytes a lane, 16 rows at a
  // time (rows step 4 banks: +16 bytes); V rows are read 8 bytes a lane by
  // groups of 16 lanes covering 4 rows x 64 bytes, two groups at a time
  // (rows step 16 banks: +64 bytes), so neither read meets a bank conflict.
  static constexpr int KPITCH = D * 2 + 16;
  static constexpr int VPITCH = D * 2 + 64;
};

__device__ __forceinline__ int row32(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <int D>
struct RowTile32Attn {
  using Sh = Tile32Shape<D>;
  static constexpr int DK = Sh::DK, DT = Sh::DT;
  static constexpr int KC = 32;  // keys per fold
  static constexpr float kLazy = 8.0f;

  bf16x8 qb[DK];  // lane l: query row l % 32, d = 16 i + 8 (l / 32) ..
  f32x16 o[DT];   // lane l, register r: row row32(l, r), d = 32 dt + l % 32
  float m, mth, l;  // this lane's row (l: over this lane's tokens only)

  __device__ __forceinline__ void reset() {
    m = kNoMax;
    mth = kNoMax;
    l = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  }

  // row_ptr(r): element pointer to query row r < 32, or nullptr (zero row:
  // finite scores, output never stored).  Rows are taken with qs's sign.
  template <class RowPtr>
  __device__ __forceinline__ void load_q(RowPtr&& row_ptr, const QScale& qs, int lane) {
    const uint16_t* p = row_ptr(lane & 31);
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      const uint4 v = p ? qs.apply(load_chunk(p + 16 * i + 8 * (lane >> 5)))
                        : make_uint4(0, 0, 0, 0);
      qb[i] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Factor of row row32(lane, r) from the lane that holds that row's state
  // (lanes 0..31 hold rows 0..31).
  __device__ __forceinline__ static float from_row(float v, int lane, int r) {
    return __int_as_float(
        __builtin_amdgcn_ds_bpermute(row32(lane, r) * 4, __float_as_int(v)));
  }

  __device__ __forceinline__ void rescale(float mn, int lane) {
    const float alpha = fast_exp2(m - mn);
    l *= alpha;
    m = mn;
    mth = mn + kLazy;
    float f[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) f[r] = from_row(alpha, lane, r);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= f[r];
  }

  // Fold 32 keys staged in LDS: K rows at kt (KPITCH bytes apart), V rows at
  // vt (VPITCH apart), token-major, every row finite.  pos0: position of the
  // first key; rowpos: this lane's row position.  With `masked` (uniform),
  // keys past the row's position are masked; without it every key is taken.
  // c: QScale::c.
  __device__ __forceinline__ void consume(const char* kt, const char* vt, int pos0, int rowpos,
                                          bool masked, float c, int lane) {
    const int hh = lane >> 5;
    f32x16 x;
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + (lane & 31) * Sh::KPITCH +
                                                         (16 * i + 8 * hh) * 2);
      x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[i], x, 0, 0, 0);
    }
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = pos0 + row32(lane, r) <= rowpos ? x[r] : -INFINITY;
    }
    float bmax = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) bmax = fmaxf(bmax, x[r]);
    bmax = fmaxf(bmax, lane_xor<32>(bmax)) * c;
    if (__builtin_amdgcn_ballot_w64(bmax > mth) != 0) rescale(fmaxf(m, bmax), lane);

    bf16x8 ph[2], pl[2];
    float sum = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int s = 0; s < 8; s += 2) {
        const float p0 = fast_exp2(fmaf(x[8 * h + s], c, -m));
        const float p1 = fast_exp2(fmaf(x[8 * h + s + 1], c, -m));
        sum += p0 + p1;
        const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
        hw[s / 2] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // high halves
        lw[s / 2] = pack_bf16x2(p0 - __uint_as_float(b0 & 0xFFFF0000u),
                                p1 - __uint_as_float(b1 & 0xFFFF0000u));
      }
      ph[h] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      pl[h] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
    l += sum;

    // O += P V.  Lane group of 16 (lane / 16 = q) reads 4 tokens x 16 d:
    // lane L of the group points at token t0 + L / 4, d c0 + 4 (L % 4), and
    // receives d c0 + L of the 4 tokens.
    const int L = lane & 15;
    const int qg = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int c0 = 32 * dt + 16 * (qg & 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x4 v[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int t0 = 16 * h + 8 * k + 4 * hh;
          const char* p = vt + (t0 + (L >> 2)) * Sh::VPITCH + (c0 + 4 * (L & 3)) * 2;
          v[k] = __builtin_bit_cast(
              bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                          (__attribute__((address_space(3))) s16x4*)(p)));
        }
        const bf16x8 b = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph[h], b, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl[h], b, o[dt], 0, 0, 0);
      }
    }
  }

  // Write the wave's state to LDS: s_acc[row][d], s_m[row], s_l[row] (row
  // sums over both halves' tokens), for the 32 rows.
  __device__ __forceinline__ void to_lds(float (*s_acc)[D], float* s_m, float* s_l,
                                         int lane) const {
    const float t = l + lane_xor<32>(l);
    if (lane < 32) {
      s_m[lane] = m;
      s_l[lane] = t;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_acc[row32(lane, r)][32 * dt + (lane & 31)] = o[dt][r];
  }

  // Normalised output: store(row, d, value) for every row < 32 and d < D.
  template <class Store>
  __device__ __forceinline__ void store_rows(Store&& store, int lane) const {
    const float t = l + lane_xor<32>(l);  // this lane's row sum (both halves' tokens)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float rs = from_row(t, lane, r);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) store(row32(lane, r), 32 * dt + (lane & 31), o[dt][r] / rs);
    }
  }
};

}  // namespace pa
