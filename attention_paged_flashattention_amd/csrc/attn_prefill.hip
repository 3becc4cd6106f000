// Causal chunked prefill over the block-paged KV cache.
//
// What the pages describe ("SM70 release profile and acceleration status":
// prompts prefilled in 4096-token chunks, each chunk attending to the pages
// written so far; "1Cat-vLLM 1.5.0" RELEASE notes, "Flash-V100 long-context
// improvements": a long-prefill GQA kernel with FP32 accumulation that packs
// several query heads onto one KV head's tensor-core work, measured in
// useful causal FLOP/s). How it is done here (gfx950):
//
// * Work-group = 256 rows that share one KV head: floor(256/G) query tokens x
//   the G query heads of that KV head (GQA packing; any G up to 64, the rows
//   past the last whole token idle), 8 waves x 32 rows, two waves per SIMD.
// * The grid is ordered so that consecutive work-groups take consecutive KV
//   heads: with round-robin dispatch over the 8 XCDs, each XCD's L2 holds the
//   K/V of one head while all its work-groups stream it. Query tiles with the
//   most keys are dispatched first.
// * Keys are walked in 64-key tiles. Waves 0-3 load the FP8 tile with 128-bit
//   loads (one page id per tile), dequantize in registers and store 16-bit K
//   (token-major) and V (dimension-major) tiles in LDS, three buffers deep;
//   loads run three tiles ahead of the tile being multiplied. (16-bit caches
//   are staged by all 8 waves, 16 bytes of K and of V each.)
// * Ping-pong: waves 0-3 and 4-7 share the SIMDs and cross the same two
//   barriers per tile doing opposite work, so one wave's softmax (VALU) runs
//   under the other wave's MFMAs.
// * S^T = K Q^T on v_mfma_f32_32x32x16 (keys on M, query rows on N, Q held in
//   registers), FP32 accumulation. Keys are assigned to MFMA rows with bits 2
//   and 3 of the row index swapped, which makes each lane's S^T outputs the
//   8-key runs that the PV step needs as its B operand: P never leaves the
//   lane, and the V^T operand is one 16-byte LDS read.
// * Online softmax in exp2 units against a running reference max that may lag
//   the row max by up to 2^8: P is formed against it directly, and only when
//   a lane's partial row sum shows that some p could exceed 2^8 (wave vote)
//   is the tile's row max taken (reduced between the two lanes that share a
//   row) and, if it outgrew the reference, O rescaled and P formed again;
//   most tiles need no max at all. Only tiles that cross the causal diagonal
//   are masked.
// * P is rounded to fp16 (V from FP8 is exact in fp16) and O^T += V^T P^T runs
//   on v_mfma_f32_32x32x16_f16.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <int QT>
struct QOp32 { using T = half8; };
template <>
struct QOp32<Q_BF16> { using T = bf16x8; };

template <int QT>
__device__ __forceinline__ f32x16 mfma32_qk(typename QOp32<QT>::T a, typename QOp32<QT>::T b,
                                            f32x16 c) {
  if constexpr (QT == Q_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
}

constexpr float kNegInfP = -__builtin_inff();
// Growth of the running max (log2 units) tolerated before O and l are rescaled.
constexpr float kRescaleSlack = 8.0f;
// Partial row sum of one tile's P below which no lane's p can exceed 2^8.
constexpr float kPSumMax = 256.0f;

// MFMA row R of a 32-key block holds key kappa(R): bits 2 and 3 swapped.
__device__ __forceinline__ int kappa(int R) {
  return (R & ~12) | ((R & 4) << 1) | ((R & 8) >> 1);
}

template <int D, int FMT, int QT, int OT>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(const PrefillArgs a) {
  constexpr int ES = (FMT == KV_F16) ? 2 : 1;
  constexpr int BN = 64;                  // keys per tile
  constexpr int NBUF = 3;                 // LDS tile buffers
  constexpr int KPAD = D + 8;             // K tile row stride (16-bit elements)
  constexpr int VPAD = BN + 8;            // V tile row stride
  constexpr int KS = D / 16;              // QK k-steps (16 dims each)
  constexpr int DBLK = D / 32;            // 32-dim output blocks
  constexpr int NT = kPrefillThreads;
  // Staging threads: with FP8 caches only waves 0-3 load and dequantize the
  // tile. A wave that issues a tile's loads stalls on them for a few hundred
  // cycles (the loads miss L1); confined to one group, that stall falls at the
  // top of the group's softmax phase and the other group's matrix phase starts
  // without it.
  constexpr int NSTAGE_T = ES == 1 ? NT / 2 : NT;
  // elements per staging thread per tile (K and V): at least one 16-byte load
  constexpr int EPT = (BN * D / NSTAGE_T) * ES >= 16 ? BN * D / NSTAGE_T : 16 / ES;
  constexpr int NSTAGE = BN * D / EPT;    // staging threads (whole waves)
  constexpr int TPK = D / EPT;            // threads per key row
  constexpr int TPR = BN / EPT;           // threads per value row (dimension)
  static_assert(NSTAGE % 64 == 0 && NSTAGE <= NT, "staging uses whole waves");
  using OpT = typename QOp32<QT>::T;

  __shared__ __attribute__((aligned(16))) uint16_t sk[NBUF][BN * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t sv[NBUF][D * VPAD];

  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int TOK = kPrefillRows / G;       // query tokens per work-group
  int idx = blockIdx.x;
  const int g = idx % Hkv;
  idx /= Hkv;
  const int qb = a.q_blocks - 1 - (idx % a.q_blocks);  // heavy tiles first
  const int b = idx / a.q_blocks;

  // sequence bounds, context length and scales: scalar loads issued together
  // (read-only here; through the constant address space so that the
  // compiler does not make them vector loads each waited for in turn)
  const int q0 = ld_const(a.cu_seqlens, b);
  const int q1 = ld_const(a.cu_seqlens, b + 1);
  const int ctx = ld_const(a.context_lens, b);
  const float kscale = a.k_scale ? ld_const(a.k_scale, g) : 1.0f;
  const int qlen = q1 - q0;
  const int tok0 = qb * TOK;
  if (tok0 >= qlen) return;
  const int ntok = min(TOK, qlen - tok0);
  const int first_pos = ctx - qlen + tok0;          // position of the first row token
  const int last_pos = first_pos + ntok - 1;
  const int ntiles = last_pos / BN + 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const bool grp_b = w >= 4;              // ping-pong group: waves 0-3 (A), 4-7 (B)
  const int c32 = lane & 31, hgrp = lane >> 5;
  const int bs_log2 = a.bs_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int vg_log2 = bs_log2 < 6 ? bs_log2 : 6;
  const int32_t* btb = a.block_tables + (int64_t)b * a.max_blocks;
  const __attribute__((address_space(4))) int32_t* btb_s =
      (const __attribute__((address_space(4))) int32_t*)btb;
  const int64_t kvh = Hkv;

  const float C = a.softmax_scale * kscale * kv_fold<FMT>() * kLog2e;

  // This lane's query row (MFMA column): r = 32 w + c32 -> (token, head).
  const int r = w * 32 + c32;
  const int rtok = r / G, rh = g * G + r % G;
  const bool rvalid = rtok < ntok;
  const int rpos = first_pos + rtok;

  // A chunk longer than its context (outside the contract: q_len_b <=
  // context_lens[b]) puts rows before position 0; they see no key. When no
  // row of this tile sees one, its rows are written as zeros and nothing is
  // loaded (the block table is never indexed below 0). Rows before position
  // 0 in a tile that also has later rows get zeros from the masks (no key
  // passes them, so the row sum stays 0).
  if (last_pos < 0) {
    if (rvalid) {
      const int64_t obase = ((int64_t)(q0 + tok0 + rtok) * a.num_q_heads + rh) * D;
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          store_out<OT>(a.out, obase + 32 * db + 8 * (j >> 2) + 4 * hgrp + (j & 3), 0.0f);
    }
    return;
  }
  OpT qop[KS];
  {
    const uint16_t* qp = a.q + ((int64_t)(q0 + tok0 + rtok) * a.num_q_heads + rh) * D + 8 * hgrp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = rvalid ? __builtin_bit_cast(OpT, ld16(qp + 16 * ks)) : OpT{};
  }

  // ---- global -> register staging (threads below NSTAGE) ----
  // K: thread owns key kt, dims kd0 .. kd0 + EPT - 1.
  // V: thread owns dim vd, keys vk0 .. vk0 + EPT - 1.
  // Every staging thread issues the same loads for every tile, whatever the
  // context length: addresses of keys past the context are redirected to the
  // tile's first key (tiles past the last one reload the last tile), and the
  // data of such keys is zeroed when the tile is written to LDS. Loads that
  // never depend on a branch let the compiler wait only for the tile being
  // written, not for the loads issued since, and no stale slot -- NaN
  // included -- reaches the tiles.
  const int kt = tid / TPK, kd0 = (tid % TPK) * EPT;
  const int vd = tid / TPR, vk0 = (tid % TPR) * EPT;
  constexpr int KLD = EPT * ES / 16;      // 16-byte loads for K
  constexpr int VLD = EPT * ES / 16;      // 16-byte loads for V
  constexpr int KPL = 16 / ES;            // keys per 16-byte value load
  const bool stager = tid < NSTAGE;
  struct Stage {
    u32x4 k[KLD], v[VLD];
  };
  const bool uni = bs_log2 >= 6;          // a 64-key tile lies in one page
  const bool any_key = ctx > 0;           // else every load reads page 0 (discarded)
  const int last_t0 = (ntiles - 1) * BN;

  // Pages of >= 64 keys: a tile lies in one page, so its K and V sit at a
  // uniform base (scalar arithmetic on the page id) plus per-thread offsets
  // fixed for the whole loop; a key past the context reads the tile's first
  // key instead.
  const uint32_t koff = (uint32_t)((kt * D + kd0) * ES), koff0 = (uint32_t)(kd0 * ES);
  const uint32_t voff0 = (uint32_t)((vd << 6) * ES);

  auto load_kv = [&](Stage& R, int t0) __attribute__((always_inline)) {
    if constexpr (NSTAGE < NT) {
      if (!stager) return;
    }
    t0 = __builtin_amdgcn_readfirstlane(min(t0, last_t0));
    if (uni) {
      // one page-id load per tile, scalar (block tables are read-only here):
      // the vector-load counter does not track it, so waiting for it never
      // waits for K/V loads in flight
      const int64_t pg = (any_key ? (int64_t)btb_s[t0 >> bs_log2] : 0) * kvh + g;
      const int toff = t0 & bs_mask;
      const uint8_t* kb = a.key_cache + ((pg << bs_log2) + toff) * (int64_t)(D * ES);
      const uint8_t* vb = a.value_cache + (((pg << (bs_log2 - 6)) + (toff >> 6)) * D << 6) * (int64_t)ES;
      const uint32_t ko = t0 + kt < ctx ? koff : koff0;
#pragma unroll
      for (int x = 0; x < KLD; ++x) R.k[x] = ld16(kb + ko + 16 * x);
#pragma unroll
      for (int x = 0; x < VLD; ++x) {
        const uint32_t vo = t0 + vk0 + x * KPL < ctx ? voff0 + (uint32_t)((vk0 + x * KPL) * ES) : voff0;
        R.v[x] = ld16(vb + vo);
      }
    } else {
      const int key = t0 + kt < ctx ? t0 + kt : t0;
      const int64_t kpage = any_key ? (int64_t)btb[key >> bs_log2] : 0;
      const uint8_t* kp = a.key_cache +
          (((kpage * kvh + g) << bs_log2) + (key & bs_mask)) * (int64_t)(D * ES) + kd0 * ES;
#pragma unroll
      for (int x = 0; x < KLD; ++x) R.k[x] = ld16(kp + 16 * x);
#pragma unroll
      for (int x = 0; x < VLD; ++x) {
        const int k0 = t0 + vk0 + x * KPL < ctx ? t0 + vk0 + x * KPL : t0;
        const int64_t page = any_key ? (int64_t)btb[k0 >> bs_log2] : 0;
        const int vo = k0 & bs_mask;  // values: dimension-major inside 2^vg_log2-token groups
        const uint8_t* vp = a.value_cache +
            (((((page * kvh + g) << (bs_log2 - vg_log2)) + (vo >> vg_log2)) * D + vd) << vg_log2 |
             (vo & ((1 << vg_log2) - 1))) * (int64_t)ES;
        R.v[x] = ld16(vp);
      }
    }
  };

  // Keys at or past the context are zeroed here: K rows whole, V runs from
  // the first such key on (selects on the raw words, no branch).
  auto mask_kv = [&](Stage& R, int t0) __attribute__((always_inline)) {
    const uint32_t kmask = t0 + kt < ctx ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int x = 0; x < KLD; ++x) R.k[x] &= kmask;
#pragma unroll
    for (int x = 0; x < VLD; ++x) {
      const int nvalid = ctx - (t0 + vk0 + x * KPL);   // valid keys in this 16-byte run
      uint32_t wm[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int per = 4 / ES;                        // keys per 32-bit word
        const int nv = nvalid - i * per;
        const uint32_t part = ES == 1 ? (1u << (8 * (nv > 0 ? nv : 0) & 31)) - 1u
                                      : (nv > 0 ? 0x0000FFFFu : 0u);
        wm[i] = nv >= per ? 0xFFFFFFFFu : (nv <= 0 ? 0u : part);
      }
      R.v[x] &= u32x4{wm[0], wm[1], wm[2], wm[3]};
    }
  };

  // Key kt is stored in LDS row kappa(kt) of its 32-key block (kappa is its own
  // inverse), so the MFMA operand read of row R is unpermuted and consecutive
  // lanes hit consecutive rows.
  const int kt_row = (kt & ~31) | kappa(kt & 31);
  auto store_kv = [&](Stage R, int buf, int t0) __attribute__((always_inline)) {
    if constexpr (NSTAGE < NT) {
      if (!stager) return;
    }
    if (t0 + BN > ctx) mask_kv(R, t0);   // only the tile that crosses the context end
    uint16_t* kdst = &sk[buf][kt_row * KPAD + kd0];
    uint16_t* vdst = &sv[buf][vd * VPAD + vk0];
    if constexpr (FMT == KV_F16) {
#pragma unroll
      for (int x = 0; x < KLD; ++x) *reinterpret_cast<u32x4*>(kdst + 8 * x) = R.k[x];
#pragma unroll
      for (int x = 0; x < VLD; ++x) *reinterpret_cast<u32x4*>(vdst + 8 * x) = R.v[x];
    } else {
#pragma unroll
      for (int x = 0; x < KLD; ++x) {
        if constexpr (QT == Q_BF16) {
          *reinterpret_cast<bf16x8*>(kdst + 16 * x) = fp8x8_to_bf16x8<FMT>(R.k[x].x, R.k[x].y);
          *reinterpret_cast<bf16x8*>(kdst + 16 * x + 8) = fp8x8_to_bf16x8<FMT>(R.k[x].z, R.k[x].w);
        } else {
          *reinterpret_cast<half8*>(kdst + 16 * x) = fp8x8_to_half8<FMT>(R.k[x].x, R.k[x].y);
          *reinterpret_cast<half8*>(kdst + 16 * x + 8) = fp8x8_to_half8<FMT>(R.k[x].z, R.k[x].w);
        }
      }
#pragma unroll
      for (int x = 0; x < VLD; ++x) {
        *reinterpret_cast<half8*>(vdst + 16 * x) = fp8x8_to_half8<FMT>(R.v[x].x, R.v[x].y);
        *reinterpret_cast<half8*>(vdst + 16 * x + 8) = fp8x8_to_half8<FMT>(R.v[x].z, R.v[x].w);
      }
    }
  };

  // S^T = K Q^T for the two 32-key blocks of the tile in buffer kb. K operands
  // are read from LDS PF reads ahead of the MFMA that consumes them.
  constexpr int NQK = KS * 2;  // (ks, mb) pairs
  constexpr int PF = 4;
  f32x16 sacc[2];
  auto qk = [&](int kb) __attribute__((always_inline)) {
    const uint16_t* skb = sk[kb] + c32 * KPAD + 8 * hgrp;
    auto rd = [&](int i) {  // i = ks * 2 + mb
      return *reinterpret_cast<const OpT*>(skb + (i & 1) * 32 * KPAD + 16 * (i >> 1));
    };
    OpT ring[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) ring[i] = rd(i);
    __builtin_amdgcn_sched_barrier(0);
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const OpT kop = ring[i % PF];
      if (i + PF < NQK) ring[i % PF] = rd(i + PF);
      sacc[i & 1] = mfma32_qk<QT>(kop, qop[i >> 1], sacc[i & 1]);
      __builtin_amdgcn_sched_barrier(0);  // keep the read PF ahead of its MFMA
    }
  };

  float m = kNegInfP, l = 0.0f;
  f32x16 oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
  half8 pop[4];

  // Softmax of tile n (keys t0 .. t0+63, S in sacc) into P (fp16).
  auto softmax = [&](int t0) __attribute__((always_inline)) {
    // Keys held by this lane: block mb, register j -> MFMA row
    // R = 8 (j/4) + 4 hgrp + j%4 -> key t0 + 32 mb + kappa(R)
    //   = t0 + 32 mb + 16 (j/8) + 8 hgrp + 4 ((j/4)&1) + j%4.
    if (t0 + BN - 1 > first_pos) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = t0 + 32 * mb + 16 * (j >> 3) + 8 * hgrp + 4 * ((j >> 2) & 1) + (j & 3);
          if (key > rpos || key >= ctx) sacc[mb][j] = kNegInfP;
        }
    }
    // P = 2^(s*C - m) against the running reference m, into fp16, and this
    // lane's partial row sum of the fp16 values (two per dot2).
    auto exp_sum = [&]() __attribute__((always_inline)) -> float {
      const float muse = m == kNegInfP ? 0.0f : m;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][j], C, -muse));
          pop[mb * 2 + (j >> 3)][j & 7] = (_Float16)pv;
        }
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
      float ps0 = 0.0f, ps1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // (vector elements are copied to scalars before the bit casts: this
        // compiler reads element 0 when a bit cast takes a vector element)
        const u32x4 w = __builtin_bit_cast(u32x4, pop[i]);
        const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
        ps0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w0), one, ps0, false);
        ps1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w1), one, ps1, false);
        ps0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w2), one, ps0, false);
        ps1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w3), one, ps1, false);
      }
      return ps0 + ps1;
    };
    // Lazy rescaling without a per-tile max in the common case: O and l are
    // kept relative to a running reference m that lags the row max by at most
    // 8 (log2 units), so every p <= 2^8 (fine in fp16) and O/l is unchanged
    // by the choice of reference. P is first formed against m directly; each
    // p is at most the lane's partial sum, so sums <= 2^8 in every lane
    // settle the tile. Otherwise (and on a row's first tile) the tile's row
    // max is taken, m, O and l are moved to it if it exceeds m + 8 somewhere
    // in the wave, and P is formed again.
    const bool fresh = __any(m == kNegInfP);
    float lt = 0.0f;
    bool settled = false;
    if (!fresh) {
      lt = exp_sum();
      settled = !__any(!(lt <= kPSumMax));
    }
    if (!settled) {
      float tm = kNegInfP;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) tm = fmaxf(tm, sacc[mb][j]);
      tm = swap_max<32>(tm);
      const float mcand = fmaxf(m, tm * C);
      if (__any(mcand > m + kRescaleSlack)) {
        const float alpha = mcand == kNegInfP ? 1.0f : __builtin_amdgcn_exp2f(m - mcand);
        m = mcand;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) oacc[db] *= alpha;
      }
      // (P is formed again even when m did not move: keeping the first pass's
      // P alive across the max costs more registers than this rare pass)
      lt = exp_sum();
    }
    l += lt;
  };

  // O^T += V^T P^T with V from buffer vb, operands read PF ahead.
  auto pv = [&](int vb) __attribute__((always_inline)) {
    const uint16_t* svb = sv[vb] + c32 * VPAD + 8 * hgrp;
    auto rdv = [&](int i) {  // i = db * 4 + kk
      return *reinterpret_cast<const half8*>(svb + (i >> 2) * 32 * VPAD + 16 * (i & 3));
    };
    constexpr int NPV = DBLK * 4;
    half8 vring[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) vring[i] = rdv(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const half8 vop = vring[i % PF];
      if (i + PF < NPV) vring[i % PF] = rdv(i + PF);
      oacc[i >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pop[i & 3], oacc[i >> 2], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Ping-pong schedule. Both wave groups cross the same barriers but do
  // opposite work between them, so on every SIMD one wave runs softmax (VALU)
  // while the other runs MFMAs:
  //   phase 1 of tile n:  A softmax(n)            | B PV(n-1), QK(n)
  //   phase 2 of tile n:  A PV(n), QK(n+1)        | B softmax(n)
  // Tile n sits in LDS buffer n % 3 from phase 2 of tile n-1 (A's QK) to
  // phase 1 of tile n+1 (B's PV). Tile n+3's HBM loads are issued at the top of
  // tile n into one of two register sets; tile n+2 (loaded a tile earlier) is
  // written to buffer (n+2) % 3 in phase 2, after the barrier that retires its
  // last reader (B's PV of tile n-1).
  Stage R0, R1;
  load_kv(R0, 0);
  store_kv(R0, 0, 0);
  load_kv(R1, BN);
  if (ntiles > 1) store_kv(R1, 1, BN);
  load_kv(R0, 2 * BN);
  __syncthreads();
  if (!grp_b) qk(0);
  __syncthreads();
  // Rl receives tile n+3, Rs holds tile n+2.
  auto iteration = [&](int n, Stage& Rl, const Stage& Rs) __attribute__((always_inline)) {
    load_kv(Rl, (n + 3) * BN);
    // phase 1
    if (!grp_b) {
      softmax(n * BN);
    } else {
      if (n > 0) pv((n - 1) % NBUF);
      qk(n % NBUF);
    }
    __syncthreads();
    // phase 2 (tile n+2 is staged after each group's own work: the matrix
    // group's conversions then overlap its last MFMAs)
    if (!grp_b) {
      pv(n % NBUF);
      if (n + 1 < ntiles) qk((n + 1) % NBUF);
    } else {
      softmax(n * BN);
    }
    if (n + 2 < ntiles) store_kv(Rs, (n + 2) % NBUF, (n + 2) * BN);
    __syncthreads();
  };
  // pairs of tiles, so the loop body always issues the same loads
  int n = 0;
  for (; n + 1 < ntiles; n += 2) {
    iteration(n, R1, R0);
    iteration(n + 1, R0, R1);
  }
  if (n < ntiles) iteration(n, R1, R0);
  if (grp_b) pv((ntiles - 1) % NBUF);

  // Epilogue: lane holds O^T[d = 32 db + 8 (j/4) + 4 hgrp + j%4][row r]. The
  // normalised rows go through LDS (the tile buffers, free after the last PV)
  // so that they leave as 16-byte runs of a row: stored straight from the
  // MFMA layout, each store instruction would write 2 or 4 bytes to each of
  // 64 rows, and the wave would stall issuing 64 of them.
  l = swap_sum<32>(l);
  const float vscale = (a.v_scale ? ld_const(a.v_scale, g) : 1.0f) * kv_fold<FMT>();
  const float f = (rvalid && l > 0.0f) ? vscale / l : 0.0f;
  constexpr int OES = OT == O_F32 ? 4 : 2;             // output element bytes
  // dimensions per pass: rows of at most 256 bytes, four waves' rows within
  // each tile array
  constexpr int LIMB = (int)((sizeof(sk) < sizeof(sv) ? sizeof(sk) : sizeof(sv)) / 128) - 16;
  constexpr int DH0 = 256 / OES < D ? 256 / OES : D;
  constexpr int DH = DH0 * OES <= LIMB ? DH0 : DH0 / 2;
  constexpr int RSTRIDE = DH * OES + 16;               // LDS row stride (bytes)
  constexpr int CPR = DH * OES / 16;                   // 16-byte chunks per row
  static_assert(4 * 32 * RSTRIDE <= (int)sizeof(sk) && 4 * 32 * RSTRIDE <= (int)sizeof(sv) &&
                (32 * CPR) % 64 == 0 && D % DH == 0, "four waves' rows fit in each tile array");
  uint8_t* stage = (w < 4 ? reinterpret_cast<uint8_t*>(&sk[0][0])
                          : reinterpret_cast<uint8_t*>(&sv[0][0])) + (w & 3) * 32 * RSTRIDE;
  uint8_t* const outb = reinterpret_cast<uint8_t*>(a.out);
#pragma unroll
  for (int pass = 0; pass < D / DH; ++pass) {
    __syncthreads();   // the tile buffers (or the previous pass's rows) are no longer read
#pragma unroll
    for (int db = pass * DH / 32; db < (pass + 1) * DH / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int col = 32 * db + 8 * jj + 4 * hgrp - pass * DH;
        uint8_t* dst = stage + c32 * RSTRIDE + col * OES;
        const float v0 = oacc[db][4 * jj] * f, v1 = oacc[db][4 * jj + 1] * f;
        const float v2 = oacc[db][4 * jj + 2] * f, v3 = oacc[db][4 * jj + 3] * f;
        if constexpr (OT == O_F32) {
          *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
        } else if constexpr (OT == O_F16) {
          const _Float16 h[4] = {(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
          *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, h);
        } else {
          *reinterpret_cast<u32x2*>(dst) =
              u32x2{(uint32_t)f32_to_bf16_rne(v0) | ((uint32_t)f32_to_bf16_rne(v1) << 16),
                    (uint32_t)f32_to_bf16_rne(v2) | ((uint32_t)f32_to_bf16_rne(v3) << 16)};
        }
      }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 32 * CPR / 64; ++k) {
      const int idx = k * 64 + lane;
      const int rr = idx / CPR, ch = idx % CPR;
      const int r2 = w * 32 + rr;
      const int tk = r2 / G;
      if (tk < ntok) {
        const int64_t row = (int64_t)(q0 + tok0 + tk) * a.num_q_heads + g * G + r2 % G;
        *reinterpret_cast<u32x4*>(outb + (row * D + pass * DH) * OES + ch * 16) =
            *reinterpret_cast<const u32x4*>(stage + rr * RSTRIDE + ch * 16);
      }
    }
  }
}

template <int D, int FMT, int QT>
static hipError_t launch_pf(const PrefillArgs& a, int ot, hipStream_t s, const ProfileEvents& ev) {
  const unsigned nblk = (unsigned)((int64_t)a.num_kv_heads * a.q_blocks * a.batch);
  dim3 grid(nblk), block(kPrefillThreads);
  if (ot == O_F32) return launch_kernel(prefill_kernel<D, FMT, QT, O_F32>, grid, block, 0, s, ev, a);
  if (ot == O_F16) return launch_kernel(prefill_kernel<D, FMT, QT, O_F16>, grid, block, 0, s, ev, a);
  return launch_kernel(prefill_kernel<D, FMT, QT, O_BF16>, grid, block, 0, s, ev, a);
}

template <int D>
static hipError_t launch_pf_d(const PrefillArgs& a, int fmt, int qt, int ot, hipStream_t s,
                              const ProfileEvents& ev) {
  if (fmt == KV_F16) return launch_pf<D, KV_F16, Q_F16>(a, ot, s, ev);
  if (fmt == KV_E4M3)
    return qt == Q_BF16 ? launch_pf<D, KV_E4M3, Q_BF16>(a, ot, s, ev)
                        : launch_pf<D, KV_E4M3, Q_F16>(a, ot, s, ev);
  return qt == Q_BF16 ? launch_pf<D, KV_E5M2, Q_BF16>(a, ot, s, ev)
                      : launch_pf<D, KV_E5M2, Q_F16>(a, ot, s, ev);
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int fmt, int qt, int ot,
                          hipStream_t stream) {
  if (a.batch == 0 || a.q_blocks == 0) return hipSuccess;
  const ProfileEvents ev = take_profile_events();
  if (head_dim == 64) return launch_pf_d<64>(a, fmt, qt, ot, stream, ev);
  return launch_pf_d<128>(a, fmt, qt, ot, stream, ev);
}

}  // namespace pa
