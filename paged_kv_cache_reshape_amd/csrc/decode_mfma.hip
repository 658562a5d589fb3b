// Decode attention, fixed-size partitions, bfloat16 with large query groups
// (G = 8, 16 or 32 query heads per kv head, MQA included): q.k and p.v both
// run on the matrix cores.
//
// Why a second kernel: with G query heads per kv head every K and V byte is
// used G times, so at G >= 8 the vector-ALU kernel is bound by its multiply-
// adds, not by HBM (G flops per byte against a vector ridge near 20).  On the
// matrix cores the same work is a few instructions per 16-token tile.
//
// Same partitioning, merge and workspace as the vector-ALU kernel: one
// workgroup per kv-head group, sequence and partition; the last workgroup of
// a split sequence merges the partial states.  Per block, each wave:
//
//   1. loads K and V rows with full-row coalesced 16-byte loads (the pattern
//      that measured fastest), tokens past the context replaced by the
//      block's first token (in range, finite) -- their scores are masked;
//   2. stages them in its own LDS tile (row pitch padded by 16 bytes so that
//      the column reads below spread over the banks);
//   3. per 16-token tile and 16-head tile, S^T = K q^T with
//      v_mfma_f32_16x16x32_bf16: A = K rows (read back one token per lane),
//      B = q (held in registers), so C holds, in lane (j, n), the scores of
//      query head n against tokens 4j .. 4j+3 of the tile;
//   4. online softmax per query head in that layout (maximum over the block
//      by two lane swaps), with a lazy maximum: the kept maximum moves only
//      when a score of the block passes it by more than 8 (base 2), so every
//      weight is at most 256 and most blocks rescale nothing;
//   5. O += P V with the same MFMA: A = P (C of step 3 is already laid out as
//      an A operand: lane (j, n) holds head n, tokens 4j .. 4j+3), B = V read
//      transposed from LDS with ds_read_b64_tr_b16, which gives lane (j, n)
//      the values of tokens 4j .. 4j+3 at one d.  P is split as
//      bf16(p) + bf16(p - bf16(p)), two products, so the weights keep 16
//      significant bits (a single bf16 rounding of p would cost up to 2^-9
//      relative per weight, more than the output tolerance allows).
//
// Softmax algebra: online softmax (barellm README, paged-cache list; LLAISYS
// README, self-attention item), float32 accumulation.
#include "attn_common.hpp"

#include "decode_launch.hpp"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Buffer resource word 3 for gfx9-family raw buffer loads (32-bit data
// format; accesses are range-checked against num_records bytes).
constexpr int kBufferRsrcWord3 = 0x00020000;

// Eight waves per workgroup, no register prefetch: a wave's K and V staging
// registers and its output tiles take about 190 VGPRs, so two waves fit per
// SIMD and the second wave's loads cover the first one's arithmetic.
// Measured on MI355X (MQA batch): 8 waves without prefetch 23.9 us, 4 waves
// with one block prefetched 30.0 us.
constexpr int kGroupWaves = 8;
constexpr int kGroupPrefetch = 1;

template <int D, int BS, int G>
struct GroupShape {
  static constexpr int RL = D * 2 / 16;       // lanes per token row in a global load
  static constexpr int ROWS = 64 / RL;        // token rows per global load
  static constexpr int NI = BS / ROWS;        // global loads per block, K or V
  static constexpr int TPB = BS / 16;         // 16-token tiles per block
  static constexpr int HT = (G + 15) / 16;    // 16-head tiles
  static constexpr int DK = D / 32;           // 32-wide d chunks of q.k
  static constexpr int DT = D / 16;           // 16-wide d tiles of p.v
  static constexpr int PITCH = D * 2 + 16;    // LDS row pitch, bytes
  static constexpr int TILE = BS * PITCH;     // one of K or V, one wave
};

__device__ __forceinline__ float max4(f32x4 v) { return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])); }

// Online-softmax state of one wave for the G query heads of one kv head.
template <int D, int BS, int G>
struct GroupAttn {
  using Sh = GroupShape<D, BS, G>;
  static constexpr int TPB = Sh::TPB, HT = Sh::HT, DK = Sh::DK, DT = Sh::DT;
  static constexpr int PITCH = Sh::PITCH;
  static constexpr float kLazy = 8.0f;

  bf16x8 qb[HT][DK];  // B operand of q.k: lane (j, n) holds head 16 ht + n, d = 32 i + 8 j ..
  f32x4 o[HT][DT];    // lane (j, n): output of head 16 ht + 4 j + r at d = 16 dt + n
  float m[HT], mth[HT], l[HT];  // lane (j, n): head 16 ht + n (l: this lane's tokens only)

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

  // q_grp: q[b, first query head of the kv head, 0].
  __device__ __forceinline__ void load_q(const uint16_t* q_grp, int lane) {
    const int n = lane & 15, j = lane >> 4;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 0; i < DK; ++i) {
        const int h = 16 * ht + n;
        const uint4 v = h < G ? load_chunk(q_grp + (size_t)h * D + 32 * i + 8 * j)
                              : make_uint4(0, 0, 0, 0);
        qb[ht][i] = __builtin_bit_cast(bf16x8, v);
      }
  }

  // Rescale head tile ht to the new kept maximum mn (per lane = per head n).
  __device__ __forceinline__ void rescale(int ht, float mn, int lane) {
    const float alpha = fast_exp2(m[ht] - mn);
    l[ht] *= alpha;
    m[ht] = mn;
    mth[ht] = mn + kLazy;
    // o's register r of lane (j, n) belongs to head 4j + r: take that head's
    // factor from lane 4j + r (group 0 holds every head's factor).
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

  // One block, staged in LDS at kt / vt (rows of PITCH bytes, token-major).
  // pos0: sequence position of the block's first token.  All scores of the
  // block are formed first, so that one kept maximum per head serves every
  // weight of the block (the products below add them into the output in one
  // step).
  __device__ __forceinline__ void consume(const char* kt, const char* vt, int pos0, int ctx,
                                          bool live, float scale_log2, int lane) {
    const int n = lane & 15, j = lane >> 4;
    f32x4 x[HT][TPB];
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt) {
      bf16x8 ka[DK];
#pragma unroll
      for (int i = 0; i < DK; ++i)
        ka[i] = *reinterpret_cast<const bf16x8*>(kt + (tt * 16 + n) * PITCH + (32 * i + 8 * j) * 2);
      bool valid[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) valid[r] = live && pos0 + tt * 16 + 4 * j + r < ctx;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < DK; ++i)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i], qb[ht][i], s, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) x[ht][tt][r] = valid[r] ? s[r] * scale_log2 : -INFINITY;
      }
    }
    bf16x4 ph[HT][TPB], pl[HT][TPB];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float bmax = max4(x[ht][0]);
#pragma unroll
      for (int tt = 1; tt < TPB; ++tt) bmax = fmaxf(bmax, max4(x[ht][tt]));
      bmax = fmaxf(bmax, lane_xor<16>(bmax));
      bmax = fmaxf(bmax, lane_xor<32>(bmax));
      if (__builtin_amdgcn_ballot_w64(bmax > mth[ht]) != 0)
        rescale(ht, fmaxf(m[ht], bmax), lane);
      float sum = 0.0f;
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(x[ht][tt][r] - m[ht]);
          sum += p;
          const __bf16 hi = static_cast<__bf16>(p);
          ph[ht][tt][r] = hi;
          pl[ht][tt][r] = static_cast<__bf16>(p - static_cast<float>(hi));
        }
      l[ht] += sum;
    }
    // O += P V, one 16-wide d tile at a time; V arrives transposed from LDS.
    const int L = lane & 15;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      bf16x4 vb[TPB];
#pragma unroll
      for (int tt = 0; tt < TPB; ++tt) {
        const char* p = vt + (tt * 16 + 4 * j + (L >> 2)) * PITCH + (16 * dt + 4 * (L & 3)) * 2;
        vb[tt] = __builtin_bit_cast(
            bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(p)));
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        if constexpr (TPB == 2) {
          const bf16x8 b = __builtin_shufflevector(vb[0], vb[1], 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 ah = __builtin_shufflevector(ph[ht][0], ph[ht][1], 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 al = __builtin_shufflevector(pl[ht][0], pl[ht][1], 0, 1, 2, 3, 4, 5, 6, 7);
          o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, o[ht][dt], 0, 0, 0);
          o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, o[ht][dt], 0, 0, 0);
        } else {
          const s16x4 b = __builtin_bit_cast(s16x4, vb[0]);
          o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              __builtin_bit_cast(s16x4, ph[ht][0]), b, o[ht][dt], 0, 0, 0);
          o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              __builtin_bit_cast(s16x4, pl[ht][0]), b, o[ht][dt], 0, 0, 0);
        }
      }
    }
  }

  // Sum the per-lane token sums over the four lane groups, then write the
  // wave's state (G heads) to LDS: s_acc[h][d], s_m[h], s_l[h].
  __device__ __forceinline__ void to_lds(float (*s_acc)[D], float* s_m, float* s_l, int lane) {
    const int n = lane & 15, j = lane >> 4;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float t = l[ht];
      t += lane_xor<16>(t);
      t += lane_xor<32>(t);
      const int h = 16 * ht + n;
      if (j == 0 && h < G) {
        s_m[h] = m[ht];
        s_l[h] = t;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hh = 16 * ht + 4 * j + r;
          if (hh < G) s_acc[hh][16 * dt + n] = o[ht][dt][r];
        }
    }
  }
};

template <int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(DecodeArgs a) {
  using Sh = GroupShape<D, BS, G>;
  using T = GroupAttn<D, BS, G>;
  constexpr int RL = Sh::RL, ROWS = Sh::ROWS, NI = Sh::NI;
  constexpr int PITCH = Sh::PITCH, TILE = Sh::TILE;
  constexpr int NT = NW * 64;
  // LDS: per wave a K and a V tile while streaming; afterwards the same bytes
  // hold the waves' states for the combine.
  constexpr int kStage = NW * 2 * TILE;
  constexpr int kCombine = NW * G * (D + 2) * 4;
  __shared__ __attribute__((aligned(16))) char s_raw[kStage > kCombine ? kStage : kCombine];

  const int hpw = a.heads_per_wg;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep loops scalar
  const int Hkv = a.num_kv_heads;
  const int nwt = NW / hpw;  // waves sharing one kv head
  const int hw = wave % hpw;
  const int tw = wave / hpw;

  T st;
  PartitionWork w;
  if (!partition_prologue<BF16, D, BS, G, NT>(a, lane, w, [&](int b, int gg) {
        st.load_q(static_cast<const uint16_t*>(a.q) +
                      ((size_t)b * a.num_q_heads + (size_t)(gg * hpw + hw) * G) * D,
                  lane);
      }))
    return;
  const int g = w.gg * hpw + hw;
  st.reset();

  // Global loads: lane (row, col) reads 16 bytes at d = 8 col of token
  // i * ROWS + row of the block (load i); tokens at or past the context read
  // the block's token 0 instead.
  const int row = lane / RL, col = lane % RL;
  const uint32_t tok_bytes = (uint32_t)Hkv * D * 2;
  const uint32_t blk_bytes = tok_bytes * BS;
  const uint32_t head_off = (uint32_t)g * D * 2 + 16 * col;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  auto fetch = [&](int jb, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
    const size_t boff = (size_t)w.block(jb) * blk_bytes;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kbase + boff), 0, blk_bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vbase + boff), 0, blk_bytes, kBufferRsrcWord3);
    const int pos0 = (w.blk0 + jb) * BS;
    uint32_t off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * ROWS + row;
      off[i] = head_off + (pos0 + tok < w.ctx ? (uint32_t)tok * tok_bytes : 0u);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
      kr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off[i], 0, 0));
#pragma unroll
    for (int i = 0; i < NI; ++i)
      vr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off[i], 0, 0));
  };
  char* kt = s_raw + wave * 2 * TILE;
  char* vt = kt + TILE;
  auto consume = [&](int jb, bool live, const uint4 (&kr)[NI], const uint4 (&vr)[NI]) {
    // Stage the block (this wave's tile only; LDS keeps one wave's accesses
    // in order, so the reads below see these writes).
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * ROWS + row;
      *reinterpret_cast<uint4*>(kt + tok * PITCH + col * 16) = kr[i];
      *reinterpret_cast<uint4*>(vt + tok * PITCH + col * 16) = vr[i];
    }
    __builtin_amdgcn_wave_barrier();
    st.consume(kt, vt, (w.blk0 + jb) * BS, w.ctx, live, a.scale_log2, lane);
    __builtin_amdgcn_wave_barrier();
  };
  stream_blocks<NI, kGroupPrefetch>(tw, nwt, w.nblk_run, fetch, consume);

  // Staging area -> per-wave states.
  __syncthreads();
  float(*s_acc)[G][D] = reinterpret_cast<float(*)[G][D]>(s_raw);
  float(*s_m)[G] = reinterpret_cast<float(*)[G]>(s_raw + NW * G * D * 4);
  float(*s_l)[G] = reinterpret_cast<float(*)[G]>(s_raw + NW * G * (D + 1) * 4);
  st.to_lds(s_acc[wave], s_m[wave], s_l[wave], lane);
  __syncthreads();
  finish_partition<BF16, D, G, G, 1, NW>(a, w.b, w.gg, w.part, w.nparts, w.poisoned, s_acc,
                                            s_m, s_l);
}

template <int D, int BS, int G>
hipError_t launch_mfma_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_seqs * (a.num_kv_heads / a.heads_per_wg), a.max_parts);
  decode_mfma_kernel<D, BS, G, kGroupWaves><<<grid, kGroupWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

bool mfma_supported(int dtype, int D, int BS, int G) {
  return dtype == PA_DTYPE_BF16 && (D == 64 || D == 128) && (BS == 16 || BS == 32) &&
         (G == 8 || G == 16 || G == 32);
}

hipError_t launch_mfma(int D, int BS, int G, const DecodeArgs& a, hipStream_t s) {
  auto by_g = [&](auto d, auto bs) -> hipError_t {
    switch (G) {
      case 8: return launch_mfma_t<decltype(d)::value, decltype(bs)::value, 8>(a, s);
      case 16: return launch_mfma_t<decltype(d)::value, decltype(bs)::value, 16>(a, s);
      case 32: return launch_mfma_t<decltype(d)::value, decltype(bs)::value, 32>(a, s);
    }
    return hipErrorInvalidValue;
  };
  auto by_bs = [&](auto d) -> hipError_t {
    return BS == 16 ? by_g(d, IntC<16>{}) : by_g(d, IntC<32>{});
  };
  return D == 64 ? by_bs(IntC<64>{}) : by_bs(IntC<128>{});
}

}  // namespace pa
