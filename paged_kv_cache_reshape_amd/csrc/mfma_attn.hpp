// Matrix-core attention over 16-token tiles of K/V staged in LDS, shared by
// the large-group decode kernel and the prefill kernel.
//
// A wave holds NR query rows (query heads of one token for the decode;
// (token, head) pairs for the prefill) and folds one K/V block at a time
// into their online-softmax state:
//
//   * S^T = K q^T with v_mfma_f32_16x16x32_bf16: A = K rows read back from
//     LDS one token per lane, B = the query rows held in registers.  C's
//     register r in lane (j, n) is then the score of row n of the 16-row tile
//     against token 4j + r of the 16-token tile;
//   * each score is kept when its key position is at most the row's own
//     position (the decode's rows all sit at the last position; prefill rows
//     are causal), else it becomes -inf -- only in tiles where some key can
//     lie past some row (the caller says which), the others skip the test;
//   * the scale is applied inside the exponent, p = exp2(c s - m), one fused
//     multiply-add per score, with c > 0: a negative scale is carried by
//     negating q (exact in bf16) and a zero scale by zeroing q, c = 1;
//   * online softmax per row in that layout (block maximum by two lane swaps),
//     with a lazy maximum: the kept maximum moves only when a score of the
//     block passes it by more than 8 (base 2), so every weight is at most 256
//     and most blocks rescale nothing.  The algebra is the online softmax of
//     the pages (barellm README, paged-cache list; LLAISYS README,
//     self-attention item); the final division by the running sum removes the
//     choice of kept maximum;
//   * O += P V with the same MFMA: C of the first product is already laid out
//     as the A operand (lane (j, n): row n, tokens 4j .. 4j+3); V arrives
//     transposed from LDS through ds_read_b64_tr_b16, which gives lane (j, n)
//     the values of tokens 4j .. 4j+3 at one d.  P is split as hi + bf16(lo),
//     hi = p with its low 16 bits cleared (a bf16 value), lo = p - hi (exact),
//     two products, so the weights keep 16 significant bits (one bf16
//     rounding of p costs up to 2^-9 relative per weight, more than the output
//     tolerance allows).
#pragma once

#include "attn_common.hpp"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bfloat16 (nearest even), packed low-first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Buffer resource word 3 for gfx9-family raw buffer loads (32-bit data
// format; accesses are range-checked against num_records bytes).
constexpr int kBufferRsrcWord3 = kBufferWord3;
// Cache-policy operand of a buffer load that reads data once per launch:
// the non-temporal bit ("nt", bit 1 on gfx950).
constexpr int kLoadStreaming = kLoadNT;

template <int D, int BS, int NR>
struct TileShape {
  static constexpr int RL = D * 2 / 16;     // lanes per token row in a 16-byte global load
  static constexpr int ROWS = 64 / RL;      // token rows per wave-wide global load
  static constexpr int NI = BS / ROWS;      // wave-wide global loads per block, K or V
  static constexpr int TPB = BS / 16;       // 16-token tiles per block
  static constexpr int HT = (NR + 15) / 16; // 16-row tiles of query rows
  static constexpr int DK = D / 32;         // 32-wide d chunks of q.k
  static constexpr int DT = D / 16;         // 16-wide d tiles of p.v
  // LDS row pitches, bytes, chosen so that neither read pattern meets a bank
  // conflict (64 banks of 4 bytes): K rows are read 16 bytes a lane, 16 rows
  // at a time, so rows step 4 banks (+16 bytes); V rows are read 8 bytes a
  // lane, 4 lanes a row, 8 rows at a time, so rows step 8 banks (+32 bytes).
  static constexpr int KPITCH = D * 2 + 16;
  static constexpr int VPITCH = D * 2 + 32;
  static constexpr int KTILE = BS * KPITCH;  // K rows of one block
  static constexpr int VTILE = BS * VPITCH;  // V rows of one block
};

// How the query rows carry the softmax scale.  Scores are used as
// exp2(c * (q.k) - m) with c > 0; scale * log2(e) = c * sign, where the sign
// (-1 or 0) is applied to q as it is loaded: negating a bf16 value, or
// zeroing it, is exact.  A NaN scale stays in c (every output NaN).
struct QScale {
  float c;
  uint32_t mask;  // applied to q's bits: and-mask, then xor with flip
  uint32_t flip;
  __device__ __forceinline__ explicit QScale(float scale_log2) {
    if (scale_log2 < 0.0f) {
      c = -scale_log2; mask = 0xFFFFFFFFu; flip = 0x80008000u;
    } else if (scale_log2 == 0.0f) {
      c = 1.0f; mask = 0u; flip = 0u;
    } else {
      c = scale_log2; mask = 0xFFFFFFFFu; flip = 0u;
    }
  }
  __device__ __forceinline__ uint4 apply(uint4 v) const {
    return make_uint4((v.x & mask) ^ flip, (v.y & mask) ^ flip, (v.z & mask) ^ flip,
                      (v.w & mask) ^ flip);
  }
};

__device__ __forceinline__ float max4(f32x4 v) {
  return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
}

// Online-softmax state of one wave for NR query rows.
template <int D, int BS, int NR>
struct RowTileAttn {
  using Sh = TileShape<D, BS, NR>;
  static constexpr int TPB = Sh::TPB, HT = Sh::HT, DK = Sh::DK, DT = Sh::DT;
  static constexpr float kLazy = 8.0f;

  bf16x8 qb[HT][DK];  // B operand of q.k: lane (j, n) holds row 16 ht + n, d = 32 i + 8 j ..
  f32x4 o[HT][DT];    // lane (j, n): output of row 16 ht + 4 j + r at d = 16 dt + n
  float m[HT], mth[HT], l[HT];  // lane (j, n): row 16 ht + n (l: this lane's tokens only)

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      m[ht] = kNoMax;
      mth[ht] = kNoMax;
      l[ht] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[ht][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  // row_ptr(r): element pointer to query row r (D values), or nullptr for a
  // row that does not exist (it is then zero: its scores are finite and its
  // output is never stored).  The rows are taken with qs's sign.
  template <class RowPtr>
  __device__ __forceinline__ void load_q(RowPtr&& row_ptr, const QScale& qs, int lane) {
    const int n = lane & 15, j = lane >> 4;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const uint16_t* p = row_ptr(16 * ht + n);
#pragma unroll
      for (int i = 0; i < DK; ++i) {
        const uint4 v = p ? qs.apply(load_chunk(p + 32 * i + 8 * j)) : make_uint4(0, 0, 0, 0);
        qb[ht][i] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  // Rescale row tile ht to the new kept maximum mn (per lane = per row n).
  __device__ __forceinline__ void rescale(int ht, float mn, int lane) {
    const float alpha = fast_exp2(m[ht] - mn);
    l[ht] *= alpha;
    m[ht] = mn;
    mth[ht] = mn + kLazy;
    // o's register r of lane (j, n) belongs to row 4j + r: take that row's
    // factor from lane 4j + r (group 0 holds every row's factor).
    const int j = lane >> 4;
    float f[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      f[r] = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * j + r) * 4, __float_as_int(alpha)));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[ht][dt][r] *= f[r];
  }

  // A block's fold is split in phases so that a caller can overlap the
  // matrix-core products of one block with the vector work of another:
  //   qk        raw scores q.k (matrix cores)
  //   mask      causal mask (vector)
  //   rowmax    block maximum per row and the lazy rescale (vector, branch)
  //   weights   exp2, row sums and the hi/lo weight split (vector)
  //   pv        O += P V (matrix cores)
  // consume() runs them in order.
  static constexpr int NP = TPB >= 2 ? TPB / 2 : 1;  // 16-token tile pairs
  using Scores = f32x4[HT][TPB];    // lane (j, n): row n, tokens 4j .. 4j+3 of each tile
  using Weights = bf16x8[HT][NP];   // p.v's A operand, one bf16x8 per tile pair

  // K rows staged in LDS at kt (KPITCH bytes apart, token-major).
  __device__ __forceinline__ void qk(const char* kt, Scores& x, int lane) const {
    const int n = lane & 15, j = lane >> 4;
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt) {
      bf16x8 ka[DK];
#pragma unroll
      for (int i = 0; i < DK; ++i)
        ka[i] = *reinterpret_cast<const bf16x8*>(kt + (tt * 16 + n) * Sh::KPITCH +
                                                 (32 * i + 8 * j) * 2);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < DK; ++i)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i], qb[ht][i], s, 0, 0, 0);
        x[ht][tt] = s;
      }
    }
  }

  // Keys past a row's position become -inf (a row position of -1 masks all).
  __device__ __forceinline__ static void mask(Scores& x, int pos0, const int (&rowpos)[HT],
                                              int lane) {
    const int j = lane >> 4;
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt) {
      const int kp = pos0 + tt * 16 + 4 * j;  // key position of register 0
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          x[ht][tt][r] = kp + r <= rowpos[ht] ? x[ht][tt][r] : -INFINITY;
    }
  }

  // Block maximum of each row (scaled by c > 0); rescales the state when a
  // row's maximum passes the kept one by more than the lazy margin.
  __device__ __forceinline__ void rowmax(const Scores& x, float c, int lane) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float bmax = max4(x[ht][0]);
#pragma unroll
      for (int tt = 1; tt < TPB; ++tt) bmax = fmaxf(bmax, max4(x[ht][tt]));
      bmax = fmaxf(bmax, lane_xor<16>(bmax));
      bmax = fmaxf(bmax, lane_xor<32>(bmax)) * c;
      if (__builtin_amdgcn_ballot_w64(bmax > mth[ht]) != 0)
        rescale(ht, fmaxf(m[ht], bmax), lane);
    }
  }

  // p = exp2(c x - m) against the kept maximum; row sums; hi/lo split.
  __device__ __forceinline__ void weights(const Scores& x, float c, Weights& ph, Weights& pl) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float sum = 0.0f;
      uint32_t hw[TPB * 2], lw[TPB * 2];
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const float p0 = fast_exp2(fmaf(x[ht][tt][r], c, -m[ht]));
          const float p1 = fast_exp2(fmaf(x[ht][tt][r + 1], c, -m[ht]));
          sum += p0 + p1;
          const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
          hw[tt * 2 + r / 2] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // high halves
          const float l0 = p0 - __uint_as_float(b0 & 0xFFFF0000u);
          const float l1 = p1 - __uint_as_float(b1 & 0xFFFF0000u);
          lw[tt * 2 + r / 2] = pack_bf16x2(l0, l1);
        }
      l[ht] += sum;
      if constexpr (TPB >= 2) {
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          ph[ht][pp] = __builtin_bit_cast(
              bf16x8, make_uint4(hw[4 * pp], hw[4 * pp + 1], hw[4 * pp + 2], hw[4 * pp + 3]));
          pl[ht][pp] = __builtin_bit_cast(
              bf16x8, make_uint4(lw[4 * pp], lw[4 * pp + 1], lw[4 * pp + 2], lw[4 * pp + 3]));
        }
      } else {
        ph[ht][0] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], 0u, 0u));
        pl[ht][0] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], 0u, 0u));
      }
    }
  }

  // O += P V, one 16-wide d tile at a time; V rows staged in LDS at vt
  // (VPITCH bytes apart) arrive transposed.
  __device__ __forceinline__ void pv(const char* vt, const Weights& ph, const Weights& pl,
                                     int lane) {
    const int j = lane >> 4, L = lane & 15;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      bf16x4 vb[TPB];
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt) {
        const char* p =
            vt + (tt * 16 + 4 * j + (L >> 2)) * Sh::VPITCH + (16 * dt + 4 * (L & 3)) * 2;
        vb[tt] = __builtin_bit_cast(
            bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(p)));
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        if constexpr (TPB >= 2) {
#pragma unroll
          for (int pp = 0; pp < NP; ++pp) {
            const bf16x8 b =
                __builtin_shufflevector(vb[2 * pp], vb[2 * pp + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            o[ht][dt] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[ht][pp], b, o[ht][dt], 0, 0, 0);
            o[ht][dt] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[ht][pp], b, o[ht][dt], 0, 0, 0);
          }
        } else {
          const s16x4 b = __builtin_bit_cast(s16x4, vb[0]);
          const s16x8 h8 = __builtin_bit_cast(s16x8, ph[ht][0]);
          const s16x8 l8 = __builtin_bit_cast(s16x8, pl[ht][0]);
          const s16x4 ah = __builtin_shufflevector(h8, h8, 0, 1, 2, 3);
          const s16x4 al = __builtin_shufflevector(l8, l8, 0, 1, 2, 3);
          o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, b, o[ht][dt], 0, 0, 0);
          o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, b, o[ht][dt], 0, 0, 0);
        }
      }
    }
  }

  // One block, staged in LDS at kt (K rows, KPITCH bytes apart) and vt (V
  // rows, VPITCH apart), token-major, every row finite.  pos0: sequence
  // position of the block's first token; rowpos[ht]: this lane's row
  // position (lane (j, n) -> row 16 ht + n).  With `masked` (uniform), keys
  // past a row's position are masked (a row position of -1 masks all);
  // without it every key is taken, so the caller clears it only for blocks
  // that lie wholly at or before every live row's position.  c: QScale::c.
  // All scores of the block are formed first, so that one kept maximum per
  // row serves every weight of the block.
  __device__ __forceinline__ void consume(const char* kt, const char* vt, int pos0,
                                          const int (&rowpos)[HT], bool masked, float c,
                                          int lane) {
    Scores x;
    qk(kt, x, lane);
    if (masked) mask(x, pos0, rowpos, lane);
    rowmax(x, c, lane);
    Weights ph, pl;
    weights(x, c, ph, pl);
    pv(vt, ph, pl, lane);
  }

  // Row sums over all of the wave's tokens: lane (j, n) gets row 16 ht + n's.
  __device__ __forceinline__ float row_sum(int ht) const {
    float t = l[ht];
    t += lane_xor<16>(t);
    t += lane_xor<32>(t);
    return t;
  }

  // Write the wave's state to LDS: s_acc[row][d], s_m[row], s_l[row], rows < NR.
  __device__ __forceinline__ void to_lds(float (*s_acc)[D], float* s_m, float* s_l, int lane) {
    const int n = lane & 15, j = lane >> 4;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const float t = row_sum(ht);
      const int h = 16 * ht + n;
      if (j == 0 && h < NR) {
        s_m[h] = m[ht];
        s_l[h] = t;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hh = 16 * ht + 4 * j + r;
          if (hh < NR) s_acc[hh][16 * dt + n] = o[ht][dt][r];
        }
    }
  }

  // Normalised output of every row: store(row, d, value) for rows < NR.
  template <class Store>
  __device__ __forceinline__ void store_rows(Store&& store, int lane) const {
    const int n = lane & 15, j = lane >> 4;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const float t = row_sum(ht);
      float rs[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rs[r] = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * j + r) * 4, __float_as_int(t)));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * ht + 4 * j + r;
          if (row < NR) store(row, 16 * dt + n, o[ht][dt][r] / rs[r]);
        }
    }
  }
};

}  // namespace pa
