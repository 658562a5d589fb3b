// Decode attention, fixed-size partitions, bfloat16 with query groups of
// G = 4, 8, 16 or 32 query heads per kv head (MQA included): q.k and p.v both
// run on the matrix cores (mfma_attn.hpp).
//
// Why a second kernel: with G query heads per kv head every K and V byte is
// used G times, and the vector-ALU kernel's multiply-adds, dot-product
// reductions and conversions per byte grow with G until they, not HBM, set
// its time.  On the matrix cores the same work is a few instructions per
// 16-token tile; a 16-row tile with fewer than 16 live rows masks the rest.
// Measured on MI355X: the MQA batch ran 527 GB/s on the vector kernel; at
// G = 4 the Llama-3.2-shaped batch takes 61.5 against 66.3 us, and a
// head_dim-128 batch of 32 sequences 35.5 against 39.8 us (the launcher keeps
// G = 4 on the vector kernel for tables of more than 4096 tokens); at G = 2
// the Qwen3-shaped batch is faster on the vector kernel (32.8 against 33.1 us
// at best).
//
// Same partitioning, merge and workspace as the vector-ALU kernel: one
// workgroup per kv-head group, sequence and partition; the last workgroup of
// a split sequence merges the partial states.  The query rows of a wave are
// the G heads of the sequence's newest token, all at its position.  Per
// block, each wave loads K and V rows with full-row coalesced 16-byte loads
// (the pattern that measured fastest; tokens past the context read the
// block's first token, in range and finite, and are masked), marked
// non-temporal since each is read once, and stages them in its own LDS tile.
#include "mfma_attn.hpp"
#include "mfma_tile32.hpp"

#include <type_traits>

#include "decode_launch.hpp"

namespace pa {

// Eight waves per workgroup, no register prefetch: a wave's K and V staging
// registers and its output tiles take about 190 VGPRs, so two waves fit per
// SIMD and the second wave's loads cover the first one's arithmetic.
// Measured on MI355X (MQA batch): 8 waves without prefetch 23.9 us, 4 waves
// with one block prefetched 30.0 us.
constexpr int kGroupWaves = 8;
constexpr int kGroupPrefetch = 1;

template <int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(DecodeArgs a) {
  using Sh = TileShape<D, BS, G>;
  // 32 query heads over 32-token blocks: one 32-row tile and one 32-key fold
  // per block on v_mfma_f32_32x32x16_bf16 (mfma_tile32.hpp), half the
  // instructions of the 16x16x32 form for the same products.
  constexpr bool kT32 = G == 32 && BS == 32;
  using T = std::conditional_t<kT32, RowTile32Attn<D>, RowTileAttn<D, BS, G>>;
  constexpr int RL = Sh::RL, ROWS = Sh::ROWS, NI = Sh::NI;
  constexpr int KPITCH = kT32 ? Tile32Shape<D>::KPITCH : Sh::KPITCH;
  constexpr int VPITCH = kT32 ? Tile32Shape<D>::VPITCH : Sh::VPITCH;
  constexpr int KTILE = BS * KPITCH, VTILE = BS * VPITCH;
  constexpr int NT = NW * 64;
  // LDS: per wave a K and a V tile while streaming; afterwards the same bytes
  // hold the waves' states for the combine.
  constexpr int kStage = NW * (KTILE + VTILE);
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

  if (step_copy_role<BF16, D, BS, NT>(a, a.num_seqs * (a.num_kv_heads / a.heads_per_wg))) return;
  T st;
  const QScale qs(a.scale_log2);
  PartitionWork w;
  if (!partition_prologue<BF16, D, BS, G, NT>(a, lane, w, [&](int b, int gg) {
        const uint16_t* q_grp = static_cast<const uint16_t*>(a.q) +
                                ((size_t)b * a.num_q_heads + (size_t)(gg * hpw + hw) * G) * D;
        st.load_q([&](int h) { return h < G ? q_grp + (size_t)h * D : nullptr; }, qs, lane);
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
  auto fetch = [&](int jb, bool live, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
    const size_t boff = (size_t)w.block(jb) * blk_bytes;
    const uint32_t nrec = live ? blk_bytes : 0u;  // a prefetch past the end reads nothing
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kbase + boff), 0, nrec, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vbase + boff), 0, nrec, kBufferRsrcWord3);
    const int pos0 = (w.blk0 + jb) * BS;
    uint32_t off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * ROWS + row;
      off[i] = head_off + (pos0 + tok < w.ctx ? (uint32_t)tok * tok_bytes : 0u);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
      kr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off[i], 0, kLoadStreaming));
#pragma unroll
    for (int i = 0; i < NI; ++i)
      vr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off[i], 0, kLoadStreaming));
  };
  // A decode step's new token (position ctx - 1, in the last partition):
  // the wave that folds its block takes the step's K/V rows in place of what
  // it read in that slot (the copy workgroups store them).  Rows past the
  // context load the block's token 0, which is that slot when the new token
  // opens its block (tt == 0): they take the new rows too, so that no stale
  // value -- uninitialised memory, NaN included -- reaches a masked product.
  const bool step = a.new_k != nullptr && w.part == w.nparts - 1;
  const int tj = step ? (w.ctx - 1) / BS - w.blk0 : -1;  // block of the new token
  const int tt = (w.ctx - 1) % BS, tli = tt / ROWS, tlr = tt % ROWS;
  uint4 nk = make_uint4(0, 0, 0, 0), nv = nk;
  if (step) {
    const size_t src = ((size_t)w.b * Hkv + g) * D + col * 8;
    nk = load_chunk(static_cast<const uint16_t*>(a.new_k) + src);
    nv = load_chunk(static_cast<const uint16_t*>(a.new_v) + src);
  }
  char* kt = s_raw + wave * (KTILE + VTILE);
  char* vt = kt + KTILE;
  auto consume = [&](int jb, bool live, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
    if (jb == tj) {
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) {
        if (tt == 0 || (ii == tli && row == tlr)) {
          kr[ii] = nk;
          vr[ii] = nv;
        }
      }
    }
    // Stage the block (this wave's tile only; LDS keeps one wave's accesses
    // in order, so the reads below see these writes).
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = i * ROWS + row;
      *reinterpret_cast<uint4*>(kt + tok * KPITCH + col * 16) = kr[i];
      *reinterpret_cast<uint4*>(vt + tok * VPITCH + col * 16) = vr[i];
    }
    __builtin_amdgcn_wave_barrier();
    // Every existing row sits at the newest position; masked when not live.
    // Only the sequence's last block holds keys past the newest position.
    const int pos0 = (w.blk0 + jb) * BS;
    if constexpr (kT32) {
      st.consume(kt, vt, pos0, live ? w.ctx - 1 : -1, !live || pos0 + BS > w.ctx, qs.c, lane);
    } else {
      int rowpos[T::HT];
#pragma unroll
      for (int ht = 0; ht < T::HT; ++ht)
        rowpos[ht] = live && 16 * ht + (lane & 15) < G ? w.ctx - 1 : -1;
      st.consume(kt, vt, pos0, rowpos, !live || pos0 + BS > w.ctx, qs.c, lane);
    }
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
  finish_partition<BF16, D, G, G, 1, NW, 1>(a, w.b, w.gg, w.part, w.nparts, w.poisoned,
                                             s_acc, s_m, s_l);
}

template <int D, int BS, int G>
hipError_t launch_mfma_t(const DecodeArgs& a, hipStream_t stream) {
  const int copy_wgs = step_copy_workgroups(a, D, 2, kGroupWaves * 64);
  dim3 grid(a.num_seqs * (a.num_kv_heads / a.heads_per_wg) + copy_wgs, a.max_parts);
  decode_mfma_kernel<D, BS, G, kGroupWaves><<<grid, kGroupWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

bool mfma_supported(int dtype, int D, int BS, int G) {
  return dtype == PA_DTYPE_BF16 && (D == 64 || D == 128) && (BS == 16 || BS == 32) &&
         (G == 4 || G == 8 || G == 16 || G == 32);
}

hipError_t launch_mfma(int D, int BS, int G, const DecodeArgs& a, hipStream_t s) {
  auto by_g = [&](auto d, auto bs) -> hipError_t {
    switch (G) {
      case 4: return launch_mfma_t<decltype(d)::value, decltype(bs)::value, 4>(a, s);
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
