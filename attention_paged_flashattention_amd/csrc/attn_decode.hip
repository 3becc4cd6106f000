// Split-KV paged decode and grouped speculative verify, plus the log-sum-exp
// combine.
//
// What the pages describe ("1Cat-vLLM 1.5.0" RELEASE notes, "Flash-V100
// long-context improvements"): batched FP8 decode that loads each page id once
// and reuses it for the page's K and V loads, with cache loads widened to 128
// bits; long-context E4M3 decode routing at 128K/256K; and a grouped q8
// verifier that treats the seven drafts plus one of a sequence as one group
// over a single pass of the KV stream. How it is done here (gfx950):
//
// * Work-group (partition p, KV head g, sequence b), 4 waves. The partition's
//   keys are walked in 64-token tiles, tiles dealt round-robin to the waves.
// * All G query heads of KV head g and all q_len new tokens form the rows of
//   one MFMA operand (NQB blocks of 16 rows), so every K/V byte is loaded once
//   per (sequence, KV head) and shared by the whole group.
// * S^T = K Q^T with v_mfma_f32_16x16x32 (keys on M, query rows on N). Each
//   lane loads its key rows straight from HBM with 128-bit loads and
//   dequantizes them in registers; no other wave reads a tile. Decode (one
//   16-row block) keeps two tiles in registers. The verify groups (two or
//   four row blocks) have registers for one tile only: their loads go from
//   HBM straight into two wave-private LDS slots (buffer -> LDS copies, two
//   tiles ahead) and come back into registers when the tile's turn comes.
//   Keys are dealt to MFMA rows so that each lane's S^T outputs are
//   exactly the 16 keys it later feeds as the B operand of O^T += V^T P^T --
//   P never moves between lanes.
// * Values are stored dimension-major inside 64-token groups of a page, so a
//   lane's 16 keys of one head dimension are 16 contiguous bytes (the A operand
//   of the PV MFMA is one 128-bit load, no transpose) and a tile's values are
//   one contiguous 8 KiB run, like its keys.
// * Online softmax per row in exp2 units; the row max is reduced across the 4
//   lanes that share a row with two lane-swap instructions, the row sum stays
//   lane-partial until the end.
// * The 4 waves' (m, l, O) are merged through LDS, and each work-group writes
//   one partial per row; the combine kernel merges the partitions in a fixed
//   order, so results are bitwise reproducible. With a single partition the
//   work-group stores the normalised row itself and no combine runs.
// * The new tokens of a decode step can be written by the same kernel
//   (quantize-on-write fused in): the work-group whose keys hold them writes
//   them before its first load.
// * The same kernels run the draft model's non-causal sliding-window attention
//   ("1Cat-vLLM 1.5.0", "Production DFlash2 on V100"; "Flash-V100 long-context
//   improvements": prefix tiles outside the window are skipped): rows see keys
//   pos - W .. ctx - 1, and the partitions start at the first tile any row of
//   the sequence can see, so the prefix before the window is never read.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <int QT>
struct QOp { using T = half8; };
template <>
struct QOp<Q_BF16> { using T = bf16x8; };

template <int QT>
__device__ __forceinline__ f32x4 mfma_qk(typename QOp<QT>::T a, typename QOp<QT>::T b, f32x4 c) {
  if constexpr (QT == Q_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
}

// 8 consecutive key elements (dwords w0, w1 of FP8; or 4 dwords of fp16) as
// the QK operand type.
template <int FMT, int QT>
__device__ __forceinline__ typename QOp<QT>::T key_op(const uint32_t* dw) {
  if constexpr (FMT == KV_F16) {
    u32x4 r = {dw[0], dw[1], dw[2], dw[3]};
    return __builtin_bit_cast(typename QOp<QT>::T, r);  // QT is F16 here
  } else if constexpr (QT == Q_BF16) {
    return fp8x8_to_bf16x8<FMT>(dw[0], dw[1]);
  } else {
    return fp8x8_to_half8<FMT>(dw[0], dw[1]);
  }
}

template <int FMT>
__device__ __forceinline__ half8 val_op(const uint32_t* dw) {
  if constexpr (FMT == KV_F16) {
    u32x4 r = {dw[0], dw[1], dw[2], dw[3]};
    return __builtin_bit_cast(half8, r);
  } else {
    return fp8x8_to_half8<FMT>(dw[0], dw[1]);
  }
}

constexpr float kNegInf = -__builtin_inff();
typedef float f32x2 __attribute__((ext_vector_type(2)));
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (gfx9 layout: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;
// Growth of the running max (log2 units) tolerated before O and l are rescaled.
constexpr float kRescaleSlackD = 8.0f;
// Cache policy of the K/V stream loads (registers and LDS copies): non-temporal
// (the "nt" bit), read once.
constexpr int kStreamPolicy = 2;

// Raw cache bytes of one 64-key tile as one lane holds them.
template <int D, int ES>
struct DecodeTile {
  static constexpr int KDW = (D / 4) * ES / 4;  // dwords per lane per key row run
  static constexpr int DB = D / 16;             // 16-dim blocks
  static constexpr int VDW = 16 * ES / 4;       // dwords per lane per 16-key value run
  uint32_t k[4][KDW];
  uint32_t v[DB][VDW];
};

// Physical pages of the two 16-key runs a lane touches in a tile (its K run
// and its V run). With pages of >= 64 keys both are the tile's one page.
struct TilePages {
  int32_t k, v;
};

__device__ __forceinline__ u32x4 ld16_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Raw buffer descriptor over one page's bytes (base: wave-uniform; no stride;
// range checking left wide open: every offset used lies inside the page).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}

// 16 bytes at byte offset off of the buffer, non-temporal like ld16_stream.
__device__ __forceinline__ u32x4 ld16_buf(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy));
}

// N 16-byte LDS reads at addr + 1024 k (k = 0 .. N-1), and the wait for all
// of them, in one asm block: the outputs are complete when the block ends.
template <int N>
__device__ __forceinline__ void lds_read_tile(u32x4 (&r)[N], uint32_t addr);

template <>
__device__ __forceinline__ void lds_read_tile<16>(u32x4 (&r)[16], uint32_t addr) {
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %16 offset:1024\n"
      "ds_read_b128 %2, %16 offset:2048\n"
      "ds_read_b128 %3, %16 offset:3072\n"
      "ds_read_b128 %4, %16 offset:4096\n"
      "ds_read_b128 %5, %16 offset:5120\n"
      "ds_read_b128 %6, %16 offset:6144\n"
      "ds_read_b128 %7, %16 offset:7168\n"
      "ds_read_b128 %8, %16 offset:8192\n"
      "ds_read_b128 %9, %16 offset:9216\n"
      "ds_read_b128 %10, %16 offset:10240\n"
      "ds_read_b128 %11, %16 offset:11264\n"
      "ds_read_b128 %12, %16 offset:12288\n"
      "ds_read_b128 %13, %16 offset:13312\n"
      "ds_read_b128 %14, %16 offset:14336\n"
      "ds_read_b128 %15, %16 offset:15360\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
        "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(addr)
      : "memory");
}

template <>
__device__ __forceinline__ void lds_read_tile<8>(u32x4 (&r)[8], uint32_t addr) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %8 offset:1024\n"
      "ds_read_b128 %2, %8 offset:2048\n"
      "ds_read_b128 %3, %8 offset:3072\n"
      "ds_read_b128 %4, %8 offset:4096\n"
      "ds_read_b128 %5, %8 offset:5120\n"
      "ds_read_b128 %6, %8 offset:6144\n"
      "ds_read_b128 %7, %8 offset:7168\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(addr)
      : "memory");
}

// Fused quantize-on-write: new tokens i0 .. i1-1 of sequence b (positions
// p0 + i) for KV head g, written into the caches with the same encoding as the
// write kernels (a 16-byte source chunk -> 8 codes per thread and task). Each
// key row chunk is one 8-byte store (16 for fp16); the 8 value codes of a chunk
// go to 8 dimension rows of the token's value group.
template <int D, int FMT, int QT>
__device__ __forceinline__ void append_new_tokens(const DecodeArgs& a, int b, int g, int p0,
                                                  int i0, int i1, const int32_t* btb, int tid,
                                                  int nthreads) {
  constexpr int ES = (FMT == KV_F16) ? 2 : 1;
  constexpr int CH = D / 8;                   // 16-byte source chunks per row
  const bool ksc = a.k_scale != nullptr, vsc = a.v_scale != nullptr;
  const float kdiv = ksc ? ld_const(a.k_scale, g) : 1.0f;
  const float vdiv = vsc ? ld_const(a.v_scale, g) : 1.0f;
  const Divisor kd = make_divisor(kdiv), vd = make_divisor(vdiv);
  const int bs_log2 = a.bs_log2;
  const int vg_log2 = bs_log2 < 6 ? bs_log2 : 6;
  const int64_t T = (int64_t)1 << vg_log2;
  const int tasks = (i1 - i0) * 2 * CH;
  for (int e = tid; e < tasks; e += nthreads) {
    const int i = i0 + e / (2 * CH);
    const int r = e % (2 * CH);
    const bool isv = r >= CH;
    const int ch = isv ? r - CH : r;
    const int pos = p0 + i;
    const uint16_t* src = (isv ? a.v_new : a.k_new) +
                          ((int64_t)(b * a.q_len + i) * a.num_kv_heads + g) * D + ch * 8;
    const u32x4 w = ld16(src);
    const int64_t page = btb[pos >> bs_log2];
    const int64_t off = pos & ((1 << bs_log2) - 1);
    const int64_t ph = page * a.num_kv_heads + g;
    const u32x4 codes = isv ? encode8<QT, FMT>(w, vsc, vd)
                            : encode8<QT, FMT>(w, ksc, kd);
    if (!isv) {
      uint8_t* kdst = a.key_cache_w + (((ph << bs_log2) + off) * D + ch * 8) * ES;
      if constexpr (ES == 2) *reinterpret_cast<u32x4*>(kdst) = codes;
      else *reinterpret_cast<u32x2*>(kdst) = u32x2{codes.x, codes.y};
    } else {
      uint8_t* vdst = a.value_cache_w +
          ((((ph << (bs_log2 - vg_log2)) + (off >> vg_log2)) * D + ch * 8) * T + (off & (T - 1))) * ES;
      const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if constexpr (ES == 2)
          reinterpret_cast<uint16_t*>(vdst)[(int64_t)k * T] = (uint16_t)(cw[k >> 1] >> ((k & 1) * 16));
        else
          vdst[(int64_t)k * T] = (uint8_t)(cw[k >> 2] >> ((k & 3) * 8));
      }
    }
  }
}

// UNI: block_size >= 64, so every 64-key tile lies in one page and its page id
// is wave-uniform (a scalar load).
// PIPE: two register stages (the next tile's loads in flight while this one is
// multiplied); used where both stages fit in the registers of 2 waves per SIMD
// (FP8 cache, one 16-row query block). Otherwise tiles are loaded one at a time
// and the waves of the CU overlap each other's loads.
template <int FMT, int NQB>
struct DecodePipe {
  static constexpr bool value = FMT != KV_F16 && NQB == 1;
};

// LDS-staged pipeline for the wider row groups (FP8 cache, two or four 16-row
// blocks, pages of >= 64 keys so that page ids are scalar loads), whose
// registers hold one tile but not two: each wave's tiles are
// copied from HBM straight into two wave-private LDS slots (buffer -> LDS
// loads, no registers in flight), two tiles ahead of the one being
// multiplied, and read back into registers when their turn comes.
template <int FMT, int NQB, bool UNI>
struct DecodeLdsPipe {
  static constexpr bool value = FMT != KV_F16 && NQB >= 2 && UNI;
};

// APPEND: the fused quantize-on-write of the new tokens. ONEP: a single
// partition, whose work-group stores the normalised output itself. Both are
// separate instantiations, so the other kernels carry none of their code.
template <int D, int FMT, int QT, int NQB, bool UNI, bool APPEND, bool ONEP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DecodePipe<FMT, NQB>::value ? 2 : 1)))
void decode_split_kernel(const DecodeArgs a) {
  constexpr bool PIPE = DecodePipe<FMT, NQB>::value;
  constexpr int ES = (FMT == KV_F16) ? 2 : 1;  // bytes per cache element
  constexpr int KSTEPS = D / 32;               // MFMA k-steps over the head dim
  constexpr int RUN = D / 4;                   // key elements per lane per key row
  using Tile = DecodeTile<D, ES>;
  constexpr int KDW = Tile::KDW, DB = Tile::DB, VDW = Tile::VDW;
  using OpT = typename QOp<QT>::T;

  constexpr bool LPIPE = DecodeLdsPipe<FMT, NQB, UNI>::value;
  // bytes of one wave's tile: 16 bytes per lane per 128-bit load
  constexpr int TILE_LOADS = 4 * (KDW / 4) + DB * (VDW / 4);
  constexpr int TILE_BYTES = TILE_LOADS * 1024;
  // LDS: the two tile slots of each wave (LDS pipeline) and, after the main
  // loop, the buffers that merge the 4 waves' states (in the slots' space)
  constexpr int MERGE_FLOATS = 4 * D * 17 + 2 * NQB * 4 * 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds_slots[LPIPE ? 2 * 4 * TILE_BYTES : 1];
  __shared__ float sm_own[LPIPE ? 1 : MERGE_FLOATS];
  static_assert(!LPIPE || 2 * 4 * TILE_BYTES >= MERGE_FLOATS * 4, "merge buffers fit");
  float* sm_base = LPIPE ? reinterpret_cast<float*>(lds_slots) : sm_own;
  auto sm_o = reinterpret_cast<float (*)[D][17]>(sm_base);
  // per 16-row block: each wave's (max, sum) of its rows, kept for the stores
  auto sm_m = reinterpret_cast<float (*)[4][16]>(sm_base + 4 * D * 17);
  auto sm_l = reinterpret_cast<float (*)[4][16]>(sm_base + 4 * D * 17 + NQB * 4 * 16);

  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;   // MFMA column: query row within a 16-row block
  const int qg = lane >> 4;  // MFMA k-group
  const int G = a.num_q_heads / a.num_kv_heads;
  const int rows = a.q_len * G;
  const int32_t* btb = a.block_tables + (int64_t)b * a.max_blocks;
  // With pages of >= 64 keys and no window, the block-table entries of the
  // wave's first two tiles do not depend on the context length: they are
  // loaded beside it (one round trip before the first K/V load instead of
  // two). The indices are clamped to the row, and the values are used only
  // for tiles below the context, where the clamp never acts.
  [[maybe_unused]] int32_t pre0 = 0, pre1 = 0;
  if constexpr (UNI) {
    const int t00 = p * a.part_len + (w << 6);
    pre0 = ld_const(btb, min(t00 >> a.bs_log2, a.max_blocks - 1));
    pre1 = ld_const(btb, min((t00 + 256) >> a.bs_log2, a.max_blocks - 1));
  }
  const int ctx = ld_const(a.context_lens, b);
  // Rows are causal (window < 0), or see the keys pos - window .. ctx - 1 (the
  // non-causal sliding window). With a window the partitions tile the keys
  // from the first one any row can see, rounded down to a tile: everything
  // before it is never loaded.
  const bool win = a.window >= 0;
  const int lo_seq = win ? (max(0, ctx - a.q_len - a.window) & ~63) : 0;
  const int tb = lo_seq + p * a.part_len;
  const int te = min(tb + a.part_len, ctx);
  const int ntiles = te > tb ? (te - tb + 63) >> 6 : 0;
  const int J = ntiles > w ? (ntiles - w + 3) >> 2 : 0;  // tiles of this wave: w + 4 j
  const int bs_log2 = a.bs_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int vg_log2 = bs_log2 < 6 ? bs_log2 : 6;
  const int64_t kv_heads = a.num_kv_heads;
  const int first_masked = ctx - a.q_len + 1;  // causal: smallest key some row cannot see
  const int last_lo = ctx - 1 - a.window;      // window: largest first visible key of a row

  auto tile_t0 = [&](int j) { return tb + ((w + 4 * j) << 6); };
  auto need_mask = [&](int t0) {
    return win ? (t0 + 64 > ctx || t0 < last_lo) : t0 + 64 > first_masked;
  };

  // Page ids of tile j (loaded one tile before they are used).
  auto pages = [&](int j) {
    TilePages pg;
    const int t0 = tile_t0(j);
    if constexpr (UNI) {
      pg.k = pg.v = ld_const(btb, t0 >> bs_log2);
    } else {
      // Both entries are loaded whatever the context length (indices clamped
      // to the block-table row), so the loads need not wait for it; a run
      // past the context takes page 0 instead of the entry it read.
      const int tk = t0 + 16 * (c >> 2), tv = t0 + 16 * qg;
      const int32_t rk = btb[min(tk >> bs_log2, a.max_blocks - 1)];
      const int32_t rv = btb[min(tv >> bs_log2, a.max_blocks - 1)];
      pg.k = tk < ctx ? rk : 0;
      pg.v = tv < ctx ? rv : 0;
    }
    return pg;
  };

  // Issue the 128-bit streaming loads of tile j, unconditionally: a run past
  // the context still reads a valid page (its own page, or page 0 for a run
  // whose page is beyond the block table), and compute() masks those keys by
  // select -- S to -inf, V to zero -- whatever the stale slot holds. Keeping
  // the loads unconditional lets the compiler count them exactly, so one
  // tile's loads stay in flight while another is multiplied.
  //
  // With pages of >= 64 keys the tile lies in one page: its K rows and its
  // value group are addressed from the page's base (a scalar, one buffer
  // descriptor per tile) plus per-lane 32-bit offsets fixed for the whole
  // loop. Buffer loads need no per-lane 64-bit address arithmetic, and the
  // 128K decode measured 2-4% faster with them than with global loads of the
  // same addresses and the same non-temporal hint.
  auto load = [&](Tile& T, int j, const TilePages& pg) {
    const int t0 = tile_t0(j);
    const int tk = t0 + 16 * (c >> 2);  // first key of this lane's K run
    const int tv = t0 + 16 * qg;        // first key of this lane's V run
    if constexpr (UNI) {
      const uint8_t* kb = a.key_cache + ((pg.k * kv_heads + g) << bs_log2) * (int64_t)(D * ES);
      const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb);
      const int ko = (((tk & bs_mask) + (c & 3)) * D + RUN * qg) * ES;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int x = 0; x < KDW / 4; ++x) {
          u32x4 v = ld16_buf(kr, ko + 4 * s * D * ES + 16 * x);
          T.k[s][4 * x] = v.x; T.k[s][4 * x + 1] = v.y;
          T.k[s][4 * x + 2] = v.z; T.k[s][4 * x + 3] = v.w;
        }
      // the tile's 64-token value group: [D][64] elements
      const uint8_t* vb = a.value_cache +
          ((((pg.v * kv_heads + g) << (bs_log2 - 6)) + ((t0 & bs_mask) >> 6)) * D << 6) * (int64_t)ES;
      const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb);
      const int vo = ((c << 6) | (16 * qg)) * ES;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < VDW / 4; ++x) {
          u32x4 v = ld16_buf(vr, vo + ((db * 16) << 6) * ES + 16 * x);
          T.v[db][4 * x] = v.x; T.v[db][4 * x + 1] = v.y;
          T.v[db][4 * x + 2] = v.z; T.v[db][4 * x + 3] = v.w;
        }
      return;
    }
    const uint8_t* kp = a.key_cache +
        (((pg.k * kv_heads + g) << bs_log2) + (tk & bs_mask) + (c & 3)) * (int64_t)(D * ES) +
        RUN * qg * ES;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int x = 0; x < KDW / 4; ++x) {
        u32x4 v = ld16_stream(kp + (int64_t)4 * s * D * ES + 16 * x);
        T.k[s][4 * x] = v.x; T.k[s][4 * x + 1] = v.y;
        T.k[s][4 * x + 2] = v.z; T.k[s][4 * x + 3] = v.w;
      }
    // values: dimension-major inside groups of 2^vg_log2 tokens of a page
    const int vo = tv & bs_mask;
    const uint8_t* vp = a.value_cache +
        (((((pg.v * kv_heads + g) << (bs_log2 - vg_log2)) + (vo >> vg_log2)) * D + c) << vg_log2 |
         (vo & ((1 << vg_log2) - 1))) * (int64_t)ES;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int x = 0; x < VDW / 4; ++x) {
        u32x4 v = ld16_stream(vp + ((int64_t)(db * 16) << vg_log2) * ES + 16 * x);
        T.v[db][4 * x] = v.x; T.v[db][4 * x + 1] = v.y;
        T.v[db][4 * x + 2] = v.z; T.v[db][4 * x + 3] = v.w;
      }
  };

  // LDS pipeline: the same 128-bit loads as load(), each one a buffer -> LDS
  // copy of 16 bytes per lane (lane i's bytes land at offset 16 i of the
  // load's 1 KB block of the slot), and the read-back that gives every lane
  // exactly the words load() would have given it.
  // Only real tiles are copied (j < J): where no next tile was issued, the
  // loop waits for all copies instead of all but the next tile's. Each lane's
  // offset is one register per tile for K and one for the whole loop for V;
  // the constant part of each copy's offset goes in its scalar offset.
  [[maybe_unused]] auto dma = [&](uint8_t* slot, int j, const TilePages& pg) {
    // buffer copies from the page base (the LDS pipeline runs with pages of
    // >= 64 keys only), as in load()
    const int t0 = tile_t0(j);
    const uint8_t* kb = a.key_cache + ((pg.k * kv_heads + g) << bs_log2) * (int64_t)(D * ES);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb);
    const int ko = ((((t0 + 16 * (c >> 2)) & bs_mask) + (c & 3)) * D + RUN * qg) * ES;
    int n = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int x = 0; x < KDW / 4; ++x, ++n)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kr, (__attribute__((address_space(3))) void*)(slot + n * 1024), 16,
            ko, 4 * s * D * ES + 16 * x, 0, kStreamPolicy);
    const uint8_t* vb = a.value_cache +
        ((((pg.v * kv_heads + g) << (bs_log2 - 6)) + ((t0 & bs_mask) >> 6)) * D << 6) * (int64_t)ES;
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb);
    const int vo = ((c << 6) | (16 * qg)) * ES;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int x = 0; x < VDW / 4; ++x, ++n)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vr, (__attribute__((address_space(3))) void*)(slot + n * 1024), 16,
            vo, ((db * 16) << 6) * ES + 16 * x, 0, kStreamPolicy);
  };

  // The read-back is one asm block that ends with its own wait for the
  // reads: the compiler cannot tell which slot a pending buffer -> LDS copy
  // writes, and before reads it can see it waits for every copy in flight
  // (the next tiles' too), which would drain the pipeline each tile. The
  // explicit waits in the main loop order the copies before these reads.
  [[maybe_unused]] auto unstage = [&](Tile& T, const uint8_t* slot) {
    u32x4 r[TILE_LOADS];
    const uint32_t addr =
        (uint32_t)reinterpret_cast<uintptr_t>(slot) + (uint32_t)lane * 16u;
    lds_read_tile<TILE_LOADS>(r, addr);
    int n = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int x = 0; x < KDW / 4; ++x, ++n) {
        T.k[s][4 * x] = r[n].x; T.k[s][4 * x + 1] = r[n].y;
        T.k[s][4 * x + 2] = r[n].z; T.k[s][4 * x + 3] = r[n].w;
      }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int x = 0; x < VDW / 4; ++x, ++n) {
        T.v[db][4 * x] = r[n].x; T.v[db][4 * x + 1] = r[n].y;
        T.v[db][4 * x + 2] = r[n].z; T.v[db][4 * x + 3] = r[n].w;
      }
  };

  const float C =
      a.softmax_scale * (a.k_scale ? ld_const(a.k_scale, g) : 1.0f) * kv_fold<FMT>() * kLog2e;

  // Fused quantize-on-write: the work-group whose keys hold some of the new
  // tokens writes them for its KV head before any load (no other work-group
  // reads those keys of this head). With several new tokens every wave waits
  // until its stores have reached the L2 (vmcnt 0: gfx9 counts stores there
  // too, in issue order with the loads), then the barrier orders them before
  // every wave's loads of those keys.
  if constexpr (APPEND) {
    const int p0 = ctx - a.q_len;   // position of new token 0
    const int i0 = max(0, tb - p0), i1 = min(a.q_len, te - p0);
    if (i1 - i0 == 1) {
      // One new token in this work-group's keys: only the wave whose tile
      // holds it reads its slots (K row and value codes lie in that tile), so
      // that wave writes it and no other wave waits. Its stores go out before
      // its first tile's loads (the empty asm keeps the compiler from moving
      // memory operations across), and the wave's memory operations complete
      // in order: the wait for tile j - 2 covers the stores before tile j is
      // loaded, and a token in the wave's first two tiles is waited for here.
      const int t_idx = (p0 + i0 - tb) >> 6;   // the token's tile in the partition
      if (w == (t_idx & 3)) {
        append_new_tokens<D, FMT, QT>(a, b, g, p0, i0, i1, btb, lane, 64);
        if ((t_idx >> 2) < 2) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      }
      asm volatile("" ::: "memory");
    } else if (i1 > i0) {
      append_new_tokens<D, FMT, QT>(a, b, g, p0, i0, i1, btb, threadIdx.x, 256);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    }
  }

  // Start the first tile's traffic before anything else.
  Tile A, B;
  TilePages P0{0, 0}, P1{0, 0};
  const bool pre = UNI && !win;
  if (J > 0) P0 = pre ? TilePages{pre0, pre0} : pages(0);
  if (J > 1) P1 = pre ? TilePages{pre1, pre1} : pages(1);
  [[maybe_unused]] uint8_t* slot_a = lds_slots + (LPIPE ? w * TILE_BYTES : 0);
  [[maybe_unused]] uint8_t* slot_b = lds_slots + (LPIPE ? (4 + w) * TILE_BYTES : 0);
  [[maybe_unused]] TilePages P2{0, 0};
  if constexpr (!LPIPE) {
    if (J > 0) load(A, 0, P0);
  }
  (void)B;

  // Query operands (B of S^T = K Q^T): row r = nb*16 + c, head dims
  // RUN*qg + 8j .. +7 for k-step j. Padding rows are zero.
  OpT qop[NQB][KSTEPS];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int r = nb * 16 + c;
    if (r < rows) {
      const int qi = r / G, h = g * G + r % G;
      const uint16_t* qp = a.q + ((int64_t)(b * a.q_len + qi) * a.num_q_heads + h) * D + RUN * qg;
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) qop[nb][j] = __builtin_bit_cast(OpT, ld16(qp + 8 * j));
    } else {
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) qop[nb][j] = OpT{};
    }
  }

  if constexpr (LPIPE) {
    // tiles 0 and 1 into the wave's two slots, with tile 2's page ids
    // between them as in the loop below. Issued after the query loads, so
    // that waiting for those never waits for the tiles.
    if (J > 0) {
      dma(slot_a, 0, P0);
      P2 = pages(min(2, J - 1));
      if (J > 1) dma(slot_b, 1, P1);
    }
  }

  float m[NQB], l[NQB];
  f32x4 o[NQB][DB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    m[nb] = kNegInf;
    l[nb] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[nb][db] = f32x4{0, 0, 0, 0};
  }

  auto compute = [&](Tile& T, int j) {
    const int t0 = tile_t0(j);
    const bool nm = need_mask(t0);
    if (nm) {
      const int tv = t0 + 16 * qg;
      const int nvalid = ctx - tv;
      if (nvalid < 16) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (e >= nvalid) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              if constexpr (ES == 1) T.v[db][e >> 2] &= ~(0xFFu << ((e & 3) * 8));
              else T.v[db][e >> 1] &= ~(0xFFFFu << ((e & 1) * 16));
            }
          }
        }
      }
    }
    // S^T = K Q^T: S-tile s row i of k-group qg holds key t0 + 16 qg + 4 s + i.
    f32x4 sacc[NQB][4];
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
      for (int s = 0; s < 4; ++s) sacc[nb][s] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        OpT kop = key_op<FMT, QT>(&T.k[s][kk * (8 * ES / 4)]);
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb) sacc[nb][s] = mfma_qk<QT>(kop, qop[nb][kk], sacc[nb][s]);
      }
    }
    // Each lane's maximum over its 16 scores per block. With two or more
    // blocks it is taken in the same stretch as the products (its first terms
    // are ready before the last products are; measured: q8 +3%, the draft
    // window +2-10%), and again after masking on the few tiles that mask; the
    // empty asm keeps the compiler from sinking the first one past the branch.
    // One block takes it after the mask (the same order measured no faster).
    auto lane_max = [&](int nb) {
      float tm = kNegInf;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) tm = fmaxf(tm, sacc[nb][s][i]);
      return tm;
    };
    constexpr bool kEarlyMax = NQB >= 2;
    float tmax[NQB];
    if constexpr (kEarlyMax) {
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        tmax[nb] = lane_max(nb);
        asm volatile("" : "+v"(tmax[nb]));
      }
    }
    if (nm) {
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        const int r = nb * 16 + c;
        const int pos = ctx - a.q_len + r / G;
        const int lim_lo = win ? pos - a.window : 0;
        const int lim_hi = win ? ctx - 1 : min(pos, ctx - 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t0 + 16 * qg + 4 * s + i;
            if (key > lim_hi || key < lim_lo) sacc[nb][s][i] = kNegInf;
          }
        if constexpr (kEarlyMax) tmax[nb] = lane_max(nb);
      }
    }
    if constexpr (!kEarlyMax) {
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) tmax[nb] = lane_max(nb);
    }
    // Lazy rescaling (see the prefill kernel): the reference max is raised
    // only when some row's max exceeds it by more than 2^8. Every block's
    // decision is taken before any exponential, so the common case (no
    // rescale) is one branch-free stretch in which one block's PV products
    // run on the matrix cores while the next block's softmax is issued.
    float mcand[NQB];
    bool grow[NQB];
    bool any_grow = false;
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
      const float tm = swap_max<32>(swap_max<16>(tmax[nb]));
      mcand[nb] = fmaxf(m[nb], tm * C);
      grow[nb] = __any(mcand[nb] > m[nb] + kRescaleSlackD);
      any_grow |= grow[nb];
    }
    if (any_grow) {
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        if (grow[nb]) {
          const float alpha =
              mcand[nb] == kNegInf ? 1.0f : __builtin_amdgcn_exp2f(m[nb] - mcand[nb]);
          m[nb] = mcand[nb];
          l[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[nb][db] *= alpha;
        }
      }
    }
    half8 pop[NQB][2];
    auto softmax = [&](int nb) {
      const float muse = m[nb] == kNegInf ? 0.0f : m[nb];
      float ps = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[nb][s][i], C, -muse));
          ps += pv;
          pop[nb][s >> 1][(s & 1) * 4 + i] = (_Float16)pv;
        }
      }
      l[nb] += ps;
    };
    auto pv = [&](int nb) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          half8 vop = val_op<FMT>(&T.v[db][hh * (8 * ES / 4)]);
          o[nb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[nb][hh], o[nb][db], 0, 0, 0);
        }
      }
    };
    if constexpr (NQB >= 4) {
      // Four blocks: block nb + 1's softmax is issued between block nb's PV
      // products, one product then four VALU instructions, in a scheduling
      // region of their own (the compiler otherwise issues the products in
      // runs, and the VALU work waits behind each run). With two blocks the
      // same order measured no faster, so they keep the plain order.
      softmax(0);
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        __builtin_amdgcn_sched_barrier(0);
        if (nb + 1 < NQB) {
          softmax(nb + 1);
          pv(nb);
#pragma unroll
          for (int k = 0; k < 2 * DB; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x2, 4, 0);  // four VALU
          }
        } else {
          pv(nb);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        softmax(nb);
        pv(nb);
      }
    }
  };

  if constexpr (PIPE) {
    // Two-stage pipeline: tile j+1's loads are in flight while tile j is
    // multiplied; page ids run one more tile ahead, and each has a whole
    // tile's arithmetic to arrive. Scalar page ids (UNI) are issued after the
    // tile loads before them: scalar loads complete out of order, so using
    // one waits for every scalar load in flight. Per-lane page ids are vector
    // loads, which complete in order: they go out before the previous tile's
    // loads, so waiting for them never waits for that tile. The loop body
    // issues its loads unconditionally (page-id indices clamped to the
    // wave's last tile); the last one or two tiles are peeled.
    int j = 0;
    for (; j + 2 < J; j += 2) {
      if constexpr (UNI) {
        load(B, j + 1, P1);
        P0 = pages(j + 2);
      } else {
        P0 = pages(j + 2);
        load(B, j + 1, P1);
      }
      compute(A, j);
      if constexpr (UNI) {
        load(A, j + 2, P0);
        P1 = pages(min(j + 3, J - 1));
      } else {
        P1 = pages(min(j + 3, J - 1));
        load(A, j + 2, P0);
      }
      compute(B, j + 1);
    }
    if (j + 1 < J) {
      load(B, j + 1, P1);
      compute(A, j);
      compute(B, j + 1);
    } else if (j < J) {
      compute(A, j);
    }
  } else if constexpr (LPIPE) {
    // Tile j sits in slot j % 2; once it is back in registers the slot takes
    // tile j + 2 (if there is one), so two tiles stream in while one is
    // multiplied. The compiler does not order the buffer -> LDS copies before
    // the reads of their slot, so each read is preceded by an explicit wait:
    // issued after tile j's copies are exactly tile j + 1's copies if j + 1 <
    // J and nothing otherwise (page ids are scalar loads), so waiting until
    // that many vector-memory operations remain means tile j has landed.
    constexpr int kAfter = TILE_LOADS;
    constexpr int kWaitTile = (kAfter & 15) | ((kAfter >> 4) << 14) | 0x0F70;
    static_assert(kAfter < 64, "vmcnt holds 6 bits");
    auto wait_tile = [&](int j) {
      if (j + 1 < J) __builtin_amdgcn_s_waitcnt(kWaitTile);
      else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    };
    if (J > 0) {
      for (int j = 0; j < J; j += 2) {
        wait_tile(j);
        unstage(A, slot_a);                         // (ends with its reads done)
        P0 = pages(min(j + 3, J - 1));
        if (j + 2 < J) dma(slot_a, j + 2, P2);
        compute(A, j);
        if (j + 1 >= J) break;
        wait_tile(j + 1);
        unstage(A, slot_b);
        P2 = pages(min(j + 4, J - 1));
        if (j + 3 < J) dma(slot_b, j + 3, P0);
        compute(A, j + 1);
      }
    }
    // every copy into the slots has landed before they become merge buffers
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  } else {
    // One stage; page ids one tile ahead.
    for (int j = 0; j < J; ++j) {
      if (j > 0) load(A, j, P1);
      P1 = pages(min(j + 1, J - 1));
      compute(A, j);
    }
  }

  // Merge the 4 waves' states for each 16-row block and write one partial per
  // row: (max, sum) and the unnormalised output, all relative to the max. With
  // a single partition the merged state is the whole row: it is normalised and
  // stored here (the combine's arithmetic for one partition), and no combine
  // kernel runs.
  const int64_t P = a.num_parts;
  [[maybe_unused]] const float vscale =
      ONEP ? (a.v_scale ? ld_const(a.v_scale, g) : 1.0f) * kv_fold<FMT>() : 0.0f;
  // Thread t merges 4 consecutive dimensions of a row (D / 4 threads per row,
  // 256 / (D / 4) rows per pass) and keeps them in registers until every
  // block is merged: the stores then go out as 16-byte runs after the last
  // barrier. (Four-byte stores from inside each block's merge took most of
  // the merge's time: a wave stalls issuing each store, and the next
  // barrier waits for them.)
  constexpr int GPR = D / 4;                 // 4-dimension groups per row
  constexpr int RPP = 256 / GPR;             // rows per pass
  constexpr int PASSES = 16 / RPP;           // passes per 16-row block
  static_assert(RPP * PASSES == 16, "whole rows per pass");
  const int d0 = 4 * (threadIdx.x % GPR);
  f32x4 res[NQB][PASSES];
  float resm[NQB][PASSES], resl[NQB][PASSES];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    float lf = l[nb];
    lf = swap_sum<32>(swap_sum<16>(lf));
    if (qg == 0) {
      sm_m[nb][w][c] = m[nb];
      sm_l[nb][w][c] = lf;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[w][db * 16 + 4 * qg + i][c] = o[nb][db][i];
    __syncthreads();
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int cc = ps * RPP + threadIdx.x / GPR;
      if (nb * 16 + cc >= rows) continue;
      float M = kNegInf;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm_m[nb][ww][cc]);
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      float lt = 0.0f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = sm_m[nb][ww][cc];
        if (mw == kNegInf) continue;
        const float wt = __builtin_amdgcn_exp2f(mw - M);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += wt * sm_o[ww][d0 + i][cc];
        lt += wt * sm_l[nb][ww][cc];
      }
      if constexpr (ONEP) acc *= lt > 0.0f ? vscale / lt : 0.0f;
      res[nb][ps] = acc;
      resm[nb][ps] = M;
      resl[nb][ps] = lt;
    }
    if (nb + 1 < NQB) __syncthreads();   // sm_o is rewritten by the next block
  }
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int cc = ps * RPP + threadIdx.x / GPR;
      const int r = nb * 16 + cc;
      if (r >= rows) continue;
      const int qi = r / G, h = g * G + r % G;
      const int64_t rowg = (int64_t)(b * a.q_len + qi) * a.num_q_heads + h;
      const f32x4 v = res[nb][ps];
      if constexpr (ONEP) {
        const int64_t idx = rowg * D + d0;
        if (a.out_type == O_F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + idx) = v;
        } else if (a.out_type == O_F16) {
          const _Float16 hv[4] = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + idx) =
              __builtin_bit_cast(u32x2, hv);
        } else {
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + idx) =
              u32x2{(uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16),
                    (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16)};
        }
        continue;
      }
      *reinterpret_cast<f32x4*>(a.ws_o + (rowg * P + p) * D + d0) = v;
      if (d0 == 0)
        *reinterpret_cast<f32x2*>(a.ws_ml + (rowg * P + p) * 2) = f32x2{resm[nb][ps], resl[nb][ps]};
    }
}

// One work-group of 256 threads per output row:
//   out = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p,
// over the partitions in index order; empty partitions (m_p = -inf) weigh 0.
// Times the per-head value scale. A row with no visible key is written as zeros.
// The partition weights go to LDS (one load per partition, spread over the
// threads). Thread (slice sl, dimension group dg) adds the weighted partials of
// partitions sl, sl + SL, ... for dimensions 4dg..4dg+3, kCombineBatch 16-byte
// loads at a time; slices are summed in a fixed order, so the result does not
// depend on timing.
constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 8;
constexpr int kMaxCombineParts = 4096;

__device__ __forceinline__ float block_reduce_256(float v, float* red, bool is_max) {
  // wave64 butterfly, then the 4 wave results in order
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    const float o = lane_xor(v, m);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))
                : (red[0] + red[1]) + (red[2] + red[3]);
}

template <int D, int FMT, int OT>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(const DecodeArgs a) {
  constexpr int DG = D / 4;                   // dimension groups of 4
  constexpr int SL = kCombineThreads / DG;    // partition slices (8 at D = 128, 16 at D = 64)
  __shared__ float sw[kMaxCombineParts];
  __shared__ float red[4];
  __shared__ f32x4 sacc[SL][DG];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int h = (int)(row % a.num_q_heads);
  const int g = h / G;
  const int P = a.num_parts;
  const float* ml = a.ws_ml + row * P * 2;
  const float* po = a.ws_o + row * P * D;

  // The first batch of partials does not depend on the weights: its loads
  // are issued before the max and the weights are worked out, so at the usual
  // partition counts (P <= SL * kCombineBatch) the merge costs one round trip.
  const int dg = t % DG, sl = t / DG;
  f32x4 ov[kCombineBatch];
  auto load_batch = [&](int pb) {
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const int p = pb + k * SL;
      ov[k] = p < P ? *reinterpret_cast<const f32x4*>(po + (int64_t)p * D + 4 * dg)
                    : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  load_batch(sl);
  const float vscale = (a.v_scale ? ld_const(a.v_scale, g) : 1.0f) * kv_fold<FMT>();

  float mloc = kNegInf;
  for (int p = t; p < P; p += kCombineThreads) mloc = fmaxf(mloc, ml[2 * p]);
  const float M = block_reduce_256(mloc, red, true);
  float lloc = 0.0f;
  for (int p = t; p < P; p += kCombineThreads) {
    const float mp = ml[2 * p];
    const float wt = (mp == kNegInf || M == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mp - M);
    sw[p] = wt;
    lloc += wt * ml[2 * p + 1];
  }
  const float L = block_reduce_256(lloc, red, false);   // its barriers also publish sw

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int pb = sl; pb < P; pb += SL * kCombineBatch) {
    if (pb != sl) load_batch(pb);
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const int p = pb + k * SL;
      const float wt = p < P ? sw[p] : 0.0f;
      acc += wt * ov[k];
    }
  }
  sacc[sl][dg] = acc;
  __syncthreads();
  if (sl == 0) {
    f32x4 o = sacc[0][dg];
#pragma unroll
    for (int k = 1; k < SL; ++k) o += sacc[k][dg];
    const float f = L > 0.0f ? vscale / L : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) store_out<OT>(a.out, row * D + 4 * dg + i, o[i] * f);
  }
}

template <int D, int FMT, int QT, int NQB, bool APPEND, bool ONEP>
static hipError_t launch_split_k(const DecodeArgs& a, int batch, hipStream_t stream,
                                 const ProfileEvents& ev) {
  dim3 grid((unsigned)a.num_parts, (unsigned)a.num_kv_heads, (unsigned)batch);
  if (a.bs_log2 >= 6)
    return launch_kernel(decode_split_kernel<D, FMT, QT, NQB, true, APPEND, ONEP>, grid, dim3(256),
                         0, stream, ev, a);
  return launch_kernel(decode_split_kernel<D, FMT, QT, NQB, false, APPEND, ONEP>, grid, dim3(256),
                       0, stream, ev, a);
}

// One partition (decode and q8-wide verify): the split kernel writes the
// output and the combine is not launched.
template <int D, int FMT, int QT, int NQB, bool APPEND>
static hipError_t launch_split_app(const DecodeArgs& a, int batch, hipStream_t stream,
                                   const ProfileEvents& ev) {
  if constexpr (NQB <= 2) {
    if (a.num_parts == 1) return launch_split_k<D, FMT, QT, NQB, APPEND, true>(a, batch, stream, ev);
  }
  return launch_split_k<D, FMT, QT, NQB, APPEND, false>(a, batch, stream, ev);
}

// The fused write runs in single-block kernels only (the host writes the new
// tokens with a separate kernel for wider row groups).
template <int D, int FMT, int QT, int NQB>
static hipError_t launch_split(const DecodeArgs& a, int batch, hipStream_t stream,
                               const ProfileEvents& ev) {
  if constexpr (NQB == 1) {
    if (a.k_new != nullptr) return launch_split_app<D, FMT, QT, NQB, true>(a, batch, stream, ev);
  }
  return launch_split_app<D, FMT, QT, NQB, false>(a, batch, stream, ev);
}

template <int D, int FMT, int QT>
static hipError_t launch_split_nqb(const DecodeArgs& a, int batch, int nqb, hipStream_t stream,
                                   const ProfileEvents& ev) {
  if (nqb == 1) return launch_split<D, FMT, QT, 1>(a, batch, stream, ev);
  if (nqb == 2) return launch_split<D, FMT, QT, 2>(a, batch, stream, ev);
  return launch_split<D, FMT, QT, 4>(a, batch, stream, ev);
}

template <int D, int FMT>
static hipError_t launch_combine(const DecodeArgs& a, int64_t rows, int ot, hipStream_t stream) {
  dim3 grid((unsigned)rows), block(kCombineThreads);
  const ProfileEvents none{};
  if (ot == O_F32)
    return launch_kernel(decode_combine_kernel<D, FMT, O_F32>, grid, block, 0, stream, none, a);
  if (ot == O_F16)
    return launch_kernel(decode_combine_kernel<D, FMT, O_F16>, grid, block, 0, stream, none, a);
  return launch_kernel(decode_combine_kernel<D, FMT, O_BF16>, grid, block, 0, stream, none, a);
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, int batch, int fmt, int qt, int ot,
                                  int nqb, hipStream_t stream) {
  const ProfileEvents ev = take_profile_events();
  hipError_t e;
  if (fmt == KV_F16) {
    e = launch_split_nqb<D, KV_F16, Q_F16>(a, batch, nqb, stream, ev);
  } else if (fmt == KV_E4M3) {
    e = qt == Q_BF16 ? launch_split_nqb<D, KV_E4M3, Q_BF16>(a, batch, nqb, stream, ev)
                     : launch_split_nqb<D, KV_E4M3, Q_F16>(a, batch, nqb, stream, ev);
  } else {
    e = qt == Q_BF16 ? launch_split_nqb<D, KV_E5M2, Q_BF16>(a, batch, nqb, stream, ev)
                     : launch_split_nqb<D, KV_E5M2, Q_F16>(a, batch, nqb, stream, ev);
  }
  if (e != hipSuccess) return e;
  if (a.num_parts == 1 && nqb <= 2) return hipSuccess;   // the split kernel stored the output
  const int64_t rows = (int64_t)batch * a.q_len * a.num_q_heads;
  if (fmt == KV_F16) return launch_combine<D, KV_F16>(a, rows, ot, stream);
  if (fmt == KV_E4M3) return launch_combine<D, KV_E4M3>(a, rows, ot, stream);
  return launch_combine<D, KV_E5M2>(a, rows, ot, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int batch, int head_dim, int fmt, int qt, int ot,
                         int nqb, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (head_dim == 64) return launch_decode_d<64>(a, batch, fmt, qt, ot, nqb, stream);
  return launch_decode_d<128>(a, batch, fmt, qt, ot, nqb, stream);
}

}  // namespace pa
