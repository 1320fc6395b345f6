// Batched paged MLA decode (absorbed form) for MI355X / gfx950.
//
// What is computed (FlashInfer API docs, "prims_ts_batch_decode_with_kv_cache_mla",
// layout/mask paragraph; FlashInfer issue #3131, run_func excerpt for the one-copy
// cache; FlashInfer PR #1248, Highlights, for bmm1/bmm2; vLLM "FlashInferMLAImpl",
// class attributes, for the natural-log LSE): every (query row, head) pair of a
// request takes a softmax over bmm1_scale * q.k for the request's visible cached
// rows (576 wide) and returns bmm2_scale * P.V with V the first 512 dims of the
// same rows.  All H heads share one latent KV head, so one KV tile in LDS feeds
// every pair of the request.
//
// Kernel design (one workgroup per compute unit, persistent):
//   * Work plan, on device: every workgroup scans seq_lens / qo_indptr into LDS
//     (tiles of 64 KV rows per "unit" = request x block of 128 pairs), then owns
//     an equal, contiguous range of the linearised (unit, tile) space.  A unit cut
//     by range boundaries is written as partials and merged by a second kernel.
//     No device-to-host read anywhere.
//   * Loader: each wave streams its 16 rows of the next tile straight into LDS
//     with global_load_lds_dwordx4 (16 B per lane, one page per wave per tile, so
//     the page base is a scalar); double-buffered; rows past seq_len are never
//     loaded and are zero-filled instead, so NaN in unused slots cannot leak.
//     16-byte chunks are XOR-swizzled by row to keep LDS reads conflict-free.
//   * QK^T: S^T[32 tokens x 32 pairs] per wave on v_mfma_f32_32x32x16_bf16 with
//     the KV tile as the A operand (rows permuted so the result lands directly in
//     the B-operand layout P.V needs) and the wave's 32 query pairs held in VGPRs.
//   * Softmax: exp2 domain (log2 e folded into bmm1), one pair per lane; the
//     lane halves and the two waves of a pair group exchange maxima and sums; the
//     running max is only moved (and O rescaled) when it grows by more than 2^8.
//   * P.V: O^T[512 x 32 pairs] += V^T . P^T on the same MFMA; V^T fragments come
//     from LDS through ds_read_b64_tr_b16 (bf16) / ds_read_b64_tr_b8 (fp8).
//   * fp8 E4M3FN KV is converted exactly to bf16 in registers (v_cvt_pk_f32_fp8),
//     so the MFMA path is the same and scales only enter through bmm1/bmm2.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <atomic>
#include <mutex>

#include "mla_decode.h"

namespace {

constexpr int D_QK = 576;
constexpr int D_V = 512;
constexpr int TILE = 32;          // KV rows per LDS tile
constexpr int NBUF = 4;           // tile buffers: tiles t..t+2 resident or landing, t+3 being issued
constexpr int THREADS = 256;      // 4 waves
constexpr int PAIRS_WAVE = 32;   // (row, head) pairs per wave (MFMA N dimension)
constexpr int PAIRS_BLOCK = 64;  // pairs per unit: 2 pair groups x 32
constexpr int QK_STEPS = 18;     // 16-dim MFMA steps per wave: half of 576
constexpr int ROWB_BF16 = D_QK * 2;            // 1152
constexpr int ROWB_FP8 = D_QK;                 // 576
constexpr int TILEB = TILE * ROWB_BF16;        // 36864 bytes per buffer (fp8 tiles use half)
constexpr int PLAN_INTS = MLA_MAX_BATCH + 1;
constexpr int XS_OFF = NBUF * TILEB;           // partial-logit exchange: [4 waves][4][64 lanes][16 B]
constexpr int LDS_BYTES = XS_OFF + 4 * 4096;   // 163840: the whole LDS of a CU
// The work-plan scan (prologue only) and the end-of-segment flags alias the
// tile buffers / the exchange area when those are idle.
constexpr int PLAN_SCRATCH_OFF = 0;
constexpr int SCAN_SCRATCH_OFF = PLAN_INTS * 4 + 60;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// A segment is redone with a raised reference max only when a logit beats the
// reference by more than 2^32: P and the fp32 sums stay far from overflow below.
constexpr float RESCALE_THRESHOLD = 32.0f;

static_assert(LDS_BYTES <= 163840, "LDS budget");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Params {
  const uint16_t* q;
  const uint8_t* kv;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qo_indptr;
  uint16_t* out;
  float* lse;
  float* ws_o;      // [2G][128][512] fp32 partial O (unnormalised)
  float* ws_ml;     // [2G][128][2]   partial (max in log2 units, sum)
  int32_t* ws_plan; // [0] = tiles per workgroup C, [1] = total tiles, [2 + b] = tile offset of request b
  int32_t batch;
  int32_t heads;
  int32_t q_len_fixed;
  int32_t total_q;
  int32_t bt_stride;
  int32_t grid;
  float scale_log2;  // bmm1_scale * log2(e)
  float bmm2;
  int32_t causal;
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Query rows of request b: returns q_b and sets r0 to its first row.
__device__ __forceinline__ int request_rows(const Params& p, int b, int& r0) {
  if (p.qo_indptr != nullptr) {
    const int a = p.qo_indptr[b];
    r0 = a;
    return p.qo_indptr[b + 1] - a;
  }
  r0 = b * p.q_len_fixed;
  return p.q_len_fixed;
}

// ---------------------------------------------------------------- LDS / DMA helpers

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_wave_base)
               : "memory");
}

// Same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset.
// Both bases are wave-uniform; readfirstlane pins them to SGPRs even where the
// call sits under a lane-divergent branch.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_wave_base) {
  const uint64_t sb = (uint64_t)(uintptr_t)sbase;
  const uint64_t sbu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32)) << 32);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"((const void*)(uintptr_t)sbu), "s"(m0)
               : "memory");
}

// Wave-uniform int32 load through the scalar cache (block-table entries).
__device__ __forceinline__ int load_uniform_i32(const int32_t* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" : : : "memory"); }

__device__ __forceinline__ u32x4 lds_read_b128(const uint8_t* smem, uint32_t off) {
  return *(const __attribute__((address_space(3))) u32x4*)(
      (const __attribute__((address_space(3))) uint8_t*)smem + off);
}

__device__ __forceinline__ u32x2 lds_read_b64(const uint8_t* smem, uint32_t off) {
  return *(const __attribute__((address_space(3))) u32x2*)(
      (const __attribute__((address_space(3))) uint8_t*)smem + off);
}

__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* smem, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) uint8_t*)smem + off));
}

__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* smem, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)((__attribute__((address_space(3))) uint8_t*)smem + off));
}

// Value of lane (l ^ 32): the two halves of a wave hold the two token halves of
// the same pair.  (ds_bpermute; the permlane32_swap builtin applied to one value
// twice has been folded incorrectly by the compiler.)
__device__ __forceinline__ float other_half(float v) { return __shfl_xor(v, 32, 64); }

// 8 E4M3FN bytes -> 8 bf16 (exact: every E4M3FN value is a bf16 value).
// Byte j of (lo, hi) becomes element j.  v_cvt_pk_f32_fp8 widens two codes to
// f32, v_cvt_pk_bf16_f32 narrows the pair back without rounding error.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  bf16x8 r;
  const uint32_t src[2] = {lo, hi};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2 f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)src[i], false);
    const f32x2 f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)src[i], true);
    const bf16x2 a = __builtin_convertvector(f01, bf16x2);
    const bf16x2 c = __builtin_convertvector(f23, bf16x2);
    r[4 * i + 0] = a[0];
    r[4 * i + 1] = a[1];
    r[4 * i + 2] = c[0];
    r[4 * i + 3] = c[1];
  }
  return r;
}

// ---------------------------------------------------------------- tile layout
//
// One LDS tile buffer holds 32 cache rows split in two blocks:
//   bf16: latent block [32][1024 B] at 0, RoPE block [32][128 B] at 32768;
//   fp8 : latent block [32][512 B]  at 0, RoPE block [32][64 B]  at 16384.
// A latent row is then one 64-lane x 16 B load (bf16) or half of one (fp8).
// 16-byte chunks are XOR-swizzled by row so that both operand reads are
// bank-conflict free (64 banks x 4 B):
//   * the QK^T A read: 16 lanes read the same chunk of 16 different rows;
//   * the transposed V^T read: one instruction touches 8 rows x 64 B.
//   bf16 latent: chunk ^ (((row & 3) << 2) | ((row >> 2) & 3))   (4 bits)
//   bf16 RoPE  : chunk ^ ((row >> 1) & 7)                         (3 bits)
//   fp8 latent : chunk ^ (row & 15)                               (4 bits)
//   fp8 RoPE   : chunk ^ ((row >> 2) & 3)                         (2 bits)
constexpr int ROPE_OFF_BF16 = TILE * 1024;
constexpr int ROPE_OFF_FP8 = TILE * 512;

__device__ __forceinline__ constexpr int swz_lat_bf16(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ constexpr int swz_rope_bf16(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ constexpr int swz_lat_fp8(int row) { return row & 15; }
__device__ __forceinline__ constexpr int swz_rope_fp8(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ void lds_zero16(uint8_t* smem, uint32_t off) {
  *(__attribute__((address_space(3))) u32x4*)((__attribute__((address_space(3))) uint8_t*)smem + off) =
      u32x4{0, 0, 0, 0};
}

// ---------------------------------------------------------------- work plan

// tile_off[b] = first linear tile of request b; tile_off[B] = total tiles.
// A request contributes ceil(q_b*H / 128) units of ceil(L_b / 64) tiles each.
__device__ void build_plan(const Params& p, int* tile_off, int* scan) {
  const int tid = threadIdx.x;
  const int B = p.batch;
  const int per = (B + THREADS - 1) / THREADS;
  const int b0 = min(B, tid * per);
  const int b1 = min(B, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) {
    int r0;
    const int qb = request_rows(p, b, r0);
    local += ceil_div(qb * p.heads, PAIRS_BLOCK) * ceil_div(p.seq_lens[b], TILE);
  }
  scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < THREADS; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int run = scan[tid] - local;
  for (int b = b0; b < b1; ++b) {
    int r0;
    const int qb = request_rows(p, b, r0);
    tile_off[b] = run;
    run += ceil_div(qb * p.heads, PAIRS_BLOCK) * ceil_div(p.seq_lens[b], TILE);
  }
  if (tid == THREADS - 1) tile_off[B] = scan[THREADS - 1];
  __syncthreads();
}

// ---------------------------------------------------------------- tile loader

// DMA instructions one wave issues for a full tile.
template <bool FP8>
constexpr int tile_loads() { return FP8 ? 5 : 9; }

// Start the loads of tile t of request b into the LDS buffer at byte offset buf.
// Wave w fills rows [8w, 8w+8), which always sit in one page (page_size is a
// multiple of 16), so the page base is wave-uniform.  Rows at or past seq_len are
// never read from memory (nor is their block-table entry): they are zero-filled.
// A full tile costs each wave exactly tile_loads<FP8>() DMA instructions.
template <bool FP8, int PS>
__device__ __forceinline__ void issue_tile(const Params& p, uint8_t* smem, uint32_t buf, int b, int L, int t) {
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int row0 = t * TILE + 8 * w;
  const uint32_t lds0 = lds_addr(smem);
  if (!FP8) {
    const uint32_t lat = buf + 8 * w * 1024;
    const uint32_t rope = buf + ROPE_OFF_BF16 + 8 * w * 128;
    if (row0 >= L) {
#pragma unroll
      for (int i = 0; i < 8; ++i) lds_zero16(smem, lat + i * 1024 + lane * 16);
      lds_zero16(smem, rope + lane * 16);
      return;
    }
    const int page = load_uniform_i32(p.block_tables + (size_t)b * p.bt_stride + row0 / PS);
    const uint8_t* pg = p.kv + ((size_t)page * PS + (row0 % PS)) * ROWB_BF16;
    const int nvalid = L - row0;
    // swizzles use the row's place in the tile (8w + i)
    const int rr = lane >> 3;  // RoPE: 8 lanes per row
    const uint32_t rope_off = (uint32_t)(rr * ROWB_BF16 + 1024 + (((lane & 7) ^ swz_rope_bf16(8 * w + rr)) << 4));
    if (nvalid >= 8) {
      // all 8 rows live: scalar row base, 32-bit lane offset, no branches
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dma16_s(pg + i * ROWB_BF16, (uint32_t)((lane ^ swz_lat_bf16(8 * w + i)) << 4), lds0 + lat + i * 1024);
      dma16_s(pg, rope_off, lds0 + rope);
      return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nvalid)
        dma16_s(pg + i * ROWB_BF16, (uint32_t)((lane ^ swz_lat_bf16(8 * w + i)) << 4), lds0 + lat + i * 1024);
      else lds_zero16(smem, lat + i * 1024 + lane * 16);
    }
    if (rr < nvalid) dma16_s(pg, rope_off, lds0 + rope);
    else lds_zero16(smem, rope + lane * 16);
  } else {
    const uint32_t lat = buf + 8 * w * 512;
    const uint32_t rope = buf + ROPE_OFF_FP8 + 8 * w * 64;
    if (row0 >= L) {
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_zero16(smem, lat + i * 1024 + lane * 16);
      if (lane < 32) lds_zero16(smem, rope + lane * 16);
      return;
    }
    const int page = load_uniform_i32(p.block_tables + (size_t)b * p.bt_stride + row0 / PS);
    const uint8_t* pg = p.kv + ((size_t)page * PS + (row0 % PS)) * ROWB_FP8;
    const int nvalid = L - row0;
    const int hi = lane >> 5;
    const int rr = lane >> 2;  // RoPE: 4 lanes per row, 32 lanes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 2 * i + hi;
      if (nvalid >= 8 || r < nvalid)
        dma16_s(pg + 2 * i * ROWB_FP8, (uint32_t)(hi * ROWB_FP8 + (((lane & 31) ^ swz_lat_fp8(8 * w + r)) << 4)),
                lds0 + lat + i * 1024);
      else lds_zero16(smem, lat + i * 1024 + lane * 16);
    }
    if (lane < 32) {
      if (rr < nvalid)
        dma16_s(pg, (uint32_t)(rr * ROWB_FP8 + 512 + (((lane & 3) ^ swz_rope_fp8(8 * w + rr)) << 4)), lds0 + rope);
      else lds_zero16(smem, rope + lane * 16);
    }
  }
}

// ---------------------------------------------------------------- one segment
//
// A unit is (request, block of 64 (row, head) pairs).  The four waves form two
// pair groups of 32 pairs (grp = w >> 1) times two halves (hh = w & 1):
//   * QK^T: wave (grp, hh) contracts its 32 pairs against a tile over half of
//     the 576 head dims -- latent dims [256hh, 256hh+256) and RoPE dims
//     [512+32hh, 512+32hh+32) -- in 18 MFMAs; the two halves add their fp32
//     partial logits through LDS, so both hold the full S^T of the tile;
//   * both run the same softmax, so both hold P for all 32 tokens;
//   * P.V: wave (grp, hh) accumulates O^T for output dims [256hh, 256hh+256).
// Each wave keeps half of Q (72 VGPRs) and half of O (128 accumulators).
//
// Software pipeline over tiles (4 LDS buffers), iteration t:
//   barrier A  -> tile t+1 is in LDS, tile t-1's buffer is free: issue tile t+3;
//                 read the partner's partial logits of tile t
//   softmax(t) alongside QK^T(t+1) on the matrix cores
//   barrier B  -> the partner has read this wave's exchange slot
//   write the partial logits of tile t+1; P.V(t)
// Waves whose pair group is empty run the same barrier and DMA sequence only.

// Per-lane state of an active wave.
struct SegState {
  f32x16 acc[8];   // O^T accumulators
  float m_ref;     // reference max, log2 units (identical in both halves)
  float m_max;     // largest logit seen, log2 units
  float lsum;      // this lane's share of the softmax denominator
  bool over;       // some logit beat m_ref by more than the threshold
};

template <bool FP8, int PS, bool ACTIVE>
__device__ __forceinline__ void segment_loop(const Params& p, uint8_t* smem, int b, int L, int t0, int t1,
                                             const bf16x8 (&qf)[QK_STEPS], int n_vis, SegState& st) {
  constexpr int LOADS = tile_loads<FP8>();
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int hh = w & 1;
  const int h = lane >> 5;
  auto buf_of = [&](int t) -> uint32_t { return (uint32_t)((t - t0) % NBUF) * TILEB; };

  // ---- lane-constant LDS offsets (see the tile layout above)
  // QK^T A operand: logical row (lane & 31) is read from physical row prow;
  // quartets 1 and 2 of each 16 rows are swapped so the MFMA result rows come
  // out in the token order the P.V B operand needs.
  const int lr = lane & 31;
  const int prow = (lr & 16) | (lr & 3) | ((lr & 4) << 1) | ((lr & 8) >> 1);
  const int s16 = lane & 15;
  const int g1 = (lane >> 4) & 1;
  uint32_t qa_lat, qa_rope0, qa_rope1, tr_base;
  int qs_lat, tr_sl, tr_cc, tr_z;
  if (!FP8) {
    const int sl = swz_lat_bf16(prow), sr = swz_rope_bf16(prow);
    qa_lat = prow * 1024 + 512 * hh + 16 * (h ^ (sl & 1));
    qs_lat = sl >> 1;
    qa_rope0 = ROPE_OFF_BF16 + prow * 128 + 16 * ((4 * hh + h) ^ sr);
    qa_rope1 = ROPE_OFF_BF16 + prow * 128 + 16 * ((4 * hh + 2 + h) ^ sr);
    tr_sl = s16 >> 2;
    tr_cc = 2 * g1 + ((s16 & 3) >> 1);
    tr_base = (8 * h + tr_sl) * 1024 + 512 * hh + 8 * (s16 & 1);
    tr_z = 0;
  } else {
    qa_lat = prow * 512 + 256 * hh + 8 * h;
    qs_lat = swz_lat_fp8(prow);
    const int sr = swz_rope_fp8(prow);
    qa_rope0 = ROPE_OFF_FP8 + prow * 64 + 16 * ((2 * hh) ^ sr) + 8 * h;
    qa_rope1 = ROPE_OFF_FP8 + prow * 64 + 16 * ((2 * hh + 1) ^ sr) + 8 * h;
    tr_z = s16 >> 1;
    tr_base = (8 * h + tr_z) * 512 + 256 * hh + 8 * (s16 & 1);
    tr_sl = tr_cc = 0;
  }
  const uint32_t xs_own = XS_OFF + w * 4096 + lane * 16;
  const uint32_t xs_other = XS_OFF + (w ^ 1) * 4096 + lane * 16;

  // A fragment for 16-dim step kk of this wave (0..15 latent, 16..17 RoPE)
  auto load_a = [&](uint32_t buf, int kk) -> u32x4 {
    if (FP8) {
      const uint32_t off = (kk < 16) ? buf + qa_lat + 16 * (kk ^ qs_lat) : buf + (kk == 16 ? qa_rope0 : qa_rope1);
      const u32x2 raw = lds_read_b64(smem, off);
      return u32x4{raw[0], raw[1], 0u, 0u};
    } else {
      const uint32_t off = (kk < 16) ? buf + qa_lat + 256 * (kk >> 3) + 32 * ((kk & 7) ^ qs_lat)
                                     : buf + (kk == 16 ? qa_rope0 : qa_rope1);
      return lds_read_b128(smem, off);
    }
  };
  // V^T fragment for step = c * 8 + d (chunk c of 16 tokens, dim block d of 32)
  auto load_v = [&](uint32_t buf, int step) -> u32x4 {
    const int c = step >> 3, d = step & 7;
    if (FP8) {
      const uint32_t off = buf + 16 * c * 512 + tr_base + 16 * ((2 * d + g1) ^ (8 * h + tr_z));
      const i32x2 raw = lds_read_tr8(smem, off);
      return u32x4{(uint32_t)raw[0], (uint32_t)raw[1], 0u, 0u};
    } else {
      const uint32_t off = buf + 16 * c * 1024 + tr_base + 64 * (d & 4) + 64 * ((d & 3) ^ tr_sl);
      const s16x4 lo = lds_read_tr16(smem, off + 16 * (tr_cc ^ (2 * h)));
      const s16x4 hi = lds_read_tr16(smem, off + 4 * 1024 + 16 * (tr_cc ^ (2 * h + 1)));
      return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto to_bf16 = [&](const u32x4& raw) -> bf16x8 {
    return FP8 ? fp8x8_to_bf16x8(raw[0], raw[1]) : __builtin_bit_cast(bf16x8, raw);
  };
  auto qk_partial = [&](uint32_t buf) -> f32x16 {
    f32x16 s = f32x16{};
    constexpr int GA = 4;  // A fragments read this many steps ahead
    u32x4 araw[GA];
#pragma unroll
    for (int k = 0; k < GA; ++k) araw[k] = load_a(buf, k);
#pragma unroll
    for (int k = 0; k < QK_STEPS; ++k) {
      const u32x4 cur = araw[k % GA];
      if (k + GA < QK_STEPS) araw[k % GA] = load_a(buf, k + GA);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(to_bf16(cur), qf[k], s, 0, 0, 0);
    }
    return s;
  };
  auto store_partial = [&](const f32x16& v) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(__attribute__((address_space(3))) f32x4*)((__attribute__((address_space(3))) uint8_t*)smem + xs_own +
                                                  j * 1024) = f32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
  };

  // Tile t has landed once at most the DMA ops of the n tiles issued after it
  // remain; a partial tile among them makes the count unknown, so drain.
  auto wait_tile = [&](int t, int n) {
    n = min(n, t1 - 1 - t);
    if (n <= 0 || (t + n + 1) * TILE > L) wait_vmcnt<0>();
    else if (n == 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<2 * LOADS>();
  };

  // ---- prologue: partial logits of tile t0
  wait_tile(t0, 2);
  wait_lgkm0();
  block_barrier();
  f32x16 sp = f32x16{};
  if (ACTIVE) {
    sp = qk_partial(buf_of(t0));
    store_partial(sp);
  }

  for (int t = t0; t < t1; ++t) {
    if (t + 1 < t1) wait_tile(t + 1, 1);
    wait_lgkm0();
    block_barrier();  // A
    if (t + 3 < t1) issue_tile<FP8, PS>(p, smem, buf_of(t + 3), b, L, t + 3);
    if (!ACTIVE) {
      wait_lgkm0();
      block_barrier();  // B
      continue;
    }
    // full logits of tile t: own partial + partner's
    f32x16 s = sp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 o = *(const __attribute__((address_space(3))) f32x4*)(
          (const __attribute__((address_space(3))) uint8_t*)smem + xs_other + j * 1024);
      s[4 * j] += o[0];
      s[4 * j + 1] += o[1];
      s[4 * j + 2] += o[2];
      s[4 * j + 3] += o[3];
    }
    // QK^T of the next tile (past the last tile the buffer holds stale rows;
    // the result is then unused) runs on the matrix cores under the softmax.
    const f32x16 sn = qk_partial(buf_of(t + 1));
    // ---------------- softmax (exp2 domain); value k is token 16(k>>3) + 8h + (k&7)
    const int tok0 = t * TILE + 8 * h;
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float v = s[k] * p.scale_log2;
      v = (tok0 + 16 * (k >> 3) + (k & 7)) < n_vis ? v : -INFINITY;
      s[k] = v;
      mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, other_half(mx));
    if (st.m_ref == -INFINITY) st.m_ref = mx;  // first visible tile sets the reference
    st.m_max = fmaxf(st.m_max, mx);
    st.over = st.over || (mx > st.m_ref + RESCALE_THRESHOLD);
    const float mbase = (st.m_ref == -INFINITY) ? 0.f : st.m_ref;
    bf16x8 pc0, pc1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e0 = __builtin_amdgcn_exp2f(s[j] - mbase);
      const float e1 = __builtin_amdgcn_exp2f(s[8 + j] - mbase);
      st.lsum += e0 + e1;
      pc0[j] = (__bf16)e0;
      pc1[j] = (__bf16)e1;
    }
    wait_lgkm0();
    block_barrier();  // B
    store_partial(sn);
    // ---------------- O^T (this wave's 256 dims) += V^T . P^T over the two 16-token chunks
    {
      const uint32_t buf = buf_of(t);
      constexpr int GV = 4;  // V^T fragments read this many steps ahead
      u32x4 vraw[GV];
#pragma unroll
      for (int i = 0; i < GV; ++i) vraw[i] = load_v(buf, i);
#pragma unroll
      for (int step = 0; step < 16; ++step) {
        const u32x4 cur = vraw[step % GV];
        if (step + GV < 16) vraw[step % GV] = load_v(buf, step + GV);
        st.acc[step & 7] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(to_bf16(cur), (step >> 3) ? pc1 : pc0, st.acc[step & 7], 0, 0, 0);
      }
    }
    sp = sn;
  }
}

// Returns false when the segment has to be redone: some logit beat its lane's
// reference max (the first visible tile's max) by more than 2^32.  m_seed then
// holds each lane's observed max as the new reference and the caller runs the
// segment again, which cannot overflow; O is never rescaled.
template <bool FP8, int PS>
__device__ __forceinline__ bool process_segment(const Params& p, uint8_t* smem, int b, int pb, int L, int t0, int t1,
                                                int slot, float& m_seed) {
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int grp = w >> 1;
  const int hh = w & 1;
  const int h = lane >> 5;
  const int col = lane & 31;
  int r0;
  const int qb = request_rows(p, b, r0);
  const int H = p.heads;
  const int npairs = qb * H;
  const int pair = pb * PAIRS_BLOCK + grp * PAIRS_WAVE + col;
  const bool valid = pair < npairs;
  const int qi = valid ? pair / H : 0;
  const int head = valid ? pair - qi * H : 0;
  const int n_vis = !valid ? 0 : (p.causal ? L - qb + qi + 1 : L);
  const bool active = (pb * PAIRS_BLOCK + grp * PAIRS_WAVE) < npairs;  // uniform, same for both halves

  // first three tiles in flight before the query loads
  issue_tile<FP8, PS>(p, smem, 0, b, L, t0);
  if (t0 + 1 < t1) issue_tile<FP8, PS>(p, smem, TILEB, b, L, t0 + 1);
  if (t0 + 2 < t1) issue_tile<FP8, PS>(p, smem, 2 * TILEB, b, L, t0 + 2);

  // Query fragments (B operand): lane holds pair `col`; step kk < 16 covers latent
  // dims 256hh + 16kk + 8h .. +8, steps 16, 17 RoPE dims 512 + 32hh + 16(kk-16) + 8h.
  bf16x8 qf[QK_STEPS];
  {
    const uint16_t* qrow = p.q + ((size_t)(r0 + qi) * H + head) * D_QK + 8 * h;
#pragma unroll
    for (int k = 0; k < QK_STEPS; ++k) {
      const int dim = k < 16 ? 256 * hh + 16 * k : 512 + 32 * hh + 16 * (k - 16);
      const u32x4 v = (valid && active) ? *(const u32x4*)(qrow + dim) : u32x4{0, 0, 0, 0};
      qf[k] = __builtin_bit_cast(bf16x8, v);
    }
    // Consume the loads here so no wait on them is left inside the tile loop
    // (where it would also wait for the tiles' DMA).
#pragma unroll
    for (int k = 0; k < QK_STEPS; ++k) asm volatile("" : : "v"(qf[k]));
  }

  SegState st;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.acc[i] = f32x16{};
  st.m_ref = m_seed;
  st.m_max = m_seed;
  st.lsum = 0.f;
  st.over = false;
  if (active) segment_loop<FP8, PS, true>(p, smem, b, L, t0, t1, qf, n_vis, st);
  else segment_loop<FP8, PS, false>(p, smem, b, L, t0, t1, qf, n_vis, st);

  // ---- segment end: all waves idle on LDS; one flag per wave says "redo"
  int* flags = (int*)(smem + XS_OFF);
  wait_lgkm0();
  block_barrier();
  if (lane == 0) flags[w] = __builtin_amdgcn_ballot_w64(st.over) != 0 ? 1 : 0;
  wait_lgkm0();
  block_barrier();
  if (uniform(flags[0] | flags[1] | flags[2] | flags[3]) != 0) {
    m_seed = st.m_max;
    return false;
  }

  // ---------------- epilogue: the two lane halves hold the two token halves
  float lsum = st.lsum + other_half(st.lsum);
  if (!active || !valid) return true;
  if (slot < 0) {
    const float inv = p.bmm2 / lsum;
    uint16_t* op = p.out + ((size_t)(r0 + qi) * H + head) * D_V + 256 * hh;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dim = 32 * d + 8 * q4 + 4 * h;
        u32x2 packed;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const __bf16 lo = (__bf16)(st.acc[d][4 * q4 + 2 * e] * inv);
          const __bf16 hi = (__bf16)(st.acc[d][4 * q4 + 2 * e + 1] * inv);
          packed[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *(u32x2*)(op + dim) = packed;
      }
    }
    if (p.lse != nullptr && h == 0 && hh == 0) p.lse[(size_t)(r0 + qi) * H + head] = (st.m_ref + __log2f(lsum)) * LN2;
  } else {
    const int pl = grp * PAIRS_WAVE + col;
    float* wo = p.ws_o + ((size_t)slot * PAIRS_BLOCK + pl) * D_V + 256 * hh;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dim = 32 * d + 8 * q4 + 4 * h;
        *(float4*)(wo + dim) =
            make_float4(st.acc[d][4 * q4], st.acc[d][4 * q4 + 1], st.acc[d][4 * q4 + 2], st.acc[d][4 * q4 + 3]);
      }
    }
    if (h == 0 && hh == 0) {
      float* ml = p.ws_ml + ((size_t)slot * PAIRS_BLOCK + pl) * 2;
      ml[0] = st.m_ref;
      ml[1] = lsum;
    }
  }
  return true;
}

// ---------------------------------------------------------------- decode kernel

template <bool FP8, int PS>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  // The plan lives in LDS only until this workgroup has found its starting point.
  int* tile_off = (int*)(smem + PLAN_SCRATCH_OFF);
  build_plan(p, tile_off, (int*)(smem + SCAN_SCRATCH_OFF));
  const int B = p.batch;
  const int TT = uniform(tile_off[B]);
  const int G = p.grid;
  const int C = max(1, ceil_div(TT, G));
  if (blockIdx.x == 0) {
    for (int b = threadIdx.x; b <= B; b += THREADS) p.ws_plan[2 + b] = tile_off[b];
    if (threadIdx.x == 0) {
      p.ws_plan[0] = C;
      p.ws_plan[1] = TT;
    }
  }
  // Consecutive logical workgroups sit on one XCD (dispatch is round-robin over
  // the 8 XCDs), so workgroups sharing a request's KV share an L2.
  const int i = blockIdx.x;
  const int g = (G % 8 == 0) ? ((i & 7) * (G >> 3) + (i >> 3)) : i;
  int x = g * C;
  const int end = min(TT, x + C);
  int b = 0, rel = 0;
  if (x < end) {
    int lo = 0, hi = B;  // tile_off[lo] <= x < tile_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_off[mid] <= x) lo = mid; else hi = mid;
    }
    b = lo;
    rel = x - tile_off[lo];
  }
  b = uniform(b);
  rel = uniform(rel);
  __syncthreads();  // the LDS plan is dead from here on
  bool first = true;
  while (x < end) {
    // walk the linear (unit, tile) space forward from request b
    const int L = uniform(p.seq_lens[b]);
    int r0;
    const int qb = uniform(request_rows(p, b, r0));
    const int T = ceil_div(L, TILE);
    const int units = ceil_div(qb * p.heads, PAIRS_BLOCK);
    const int pb = rel / T;
    const int t0 = rel - pb * T;
    const int t1 = min(T, t0 + (end - x));
    const bool whole = (t0 == 0 && t1 == T);
    const int slot = whole ? -1 : (first ? 2 * g : 2 * g + 1);
    float m_seed = -INFINITY;
    while (!process_segment<FP8, PS>(p, smem, b, pb, L, t0, t1, slot, m_seed)) {
    }
    x += t1 - t0;
    rel += t1 - t0;
    if (rel >= units * T) {
      ++b;
      rel = 0;
    }
    first = false;
  }
}

// ---------------------------------------------------------------- split merge

// One wave per (query row, head).  Units written whole by the decode kernel are
// skipped; for split ones: M = max_s m_s, w_s = 2^(m_s - M),
// out = bmm2 * sum w_s O_s / sum w_s l_s, lse = ln2 * (M + log2 sum w_s l_s).
__global__ __launch_bounds__(THREADS) void mla_merge_kernel(Params p) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * (THREADS / 64) + (threadIdx.x >> 6);
  const int H = p.heads;
  if (item >= p.total_q * H) return;
  const int row = item / H;
  const int head = item - row * H;
  int b;
  if (p.qo_indptr != nullptr) {
    int lo = 0, hi = p.batch;  // qo_indptr[lo] <= row < qo_indptr[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.qo_indptr[mid] <= row) lo = mid; else hi = mid;
    }
    b = lo;
  } else {
    b = row / p.q_len_fixed;
  }
  int r0;
  request_rows(p, b, r0);
  const int pair = (row - r0) * H + head;
  const int pb = pair / PAIRS_BLOCK;
  const int pl = pair - pb * PAIRS_BLOCK;
  const int C = p.ws_plan[0];
  const int T = ceil_div(p.seq_lens[b], TILE);
  const int U0 = p.ws_plan[2 + b] + pb * T;
  const int g0 = U0 / C;
  const int g1 = (U0 + T - 1) / C;
  if (g0 == g1) return;
  float M = -INFINITY;
  for (int g = g0; g <= g1; ++g) {
    const int slot = 2 * g + ((g == g0 && U0 > g0 * C) ? 1 : 0);
    M = fmaxf(M, p.ws_ml[((size_t)slot * PAIRS_BLOCK + pl) * 2]);
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float den = 0.f;
  for (int g = g0; g <= g1; ++g) {
    const int slot = 2 * g + ((g == g0 && U0 > g0 * C) ? 1 : 0);
    const float* ml = p.ws_ml + ((size_t)slot * PAIRS_BLOCK + pl) * 2;
    const float m = ml[0];
    const float wgt = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M);
    den += wgt * ml[1];
    const float4* o = (const float4*)(p.ws_o + ((size_t)slot * PAIRS_BLOCK + pl) * D_V + 8 * lane);
    const float4 a = o[0], c = o[1];
    acc[0] += wgt * a.x; acc[1] += wgt * a.y; acc[2] += wgt * a.z; acc[3] += wgt * a.w;
    acc[4] += wgt * c.x; acc[5] += wgt * c.y; acc[6] += wgt * c.z; acc[7] += wgt * c.w;
  }
  const float inv = p.bmm2 / den;
  u32x4 packed;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 lo = (__bf16)(acc[2 * e] * inv);
    const __bf16 hi = (__bf16)(acc[2 * e + 1] * inv);
    packed[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  *(u32x4*)(p.out + (size_t)item * D_V + 8 * lane) = packed;
  if (p.lse != nullptr && lane == 0) p.lse[item] = (M + __log2f(den)) * LN2;
}

// Conversion check: the exact fp8 -> bf16 widening the decode kernel uses, on
// n groups of 8 codes (test hook).
__global__ void fp8_to_bf16_kernel(const u32x2* in, bf16x8* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const u32x2 v = in[i];
    out[i] = fp8x8_to_bf16x8(v[0], v[1]);
  }
}

// ---------------------------------------------------------------- host side

constexpr int MAX_DEVICES = 64;
std::atomic<int> g_cu_count[MAX_DEVICES];
std::atomic<int> g_grid_override{0};
std::atomic<void*> g_ev_start{nullptr};
std::atomic<void*> g_ev_stop{nullptr};

int device_grid(int* grid_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MLA_ERR_NO_DEVICE;
  int cus = g_cu_count[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return MLA_ERR_NO_DEVICE;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
  }
  const int ov = g_grid_override.load(std::memory_order_relaxed);
  *grid_out = ov > 0 ? ov : cus;
  return MLA_OK;
}

struct WsLayout {
  size_t plan_off, ml_off, o_off, total;
};

WsLayout workspace_layout(int grid) {
  WsLayout l;
  auto align = [](size_t v) { return (v + 255) & ~(size_t)255; };
  l.plan_off = 0;
  l.ml_off = align((size_t)(2 + PLAN_INTS) * 4);
  l.o_off = align(l.ml_off + (size_t)2 * grid * PAIRS_BLOCK * 2 * 4);
  l.total = align(l.o_off + (size_t)2 * grid * PAIRS_BLOCK * D_V * 4);
  return l;
}

int validate(const mla_decode_dims_t* d, int32_t max_seq_len, int32_t max_q_len, bool packed) {
  if (d == nullptr) return MLA_ERR_NULL_POINTER;
  if (d->batch < 1 || d->batch > MLA_MAX_BATCH || max_seq_len < 1 || d->num_pages < 1) return MLA_ERR_BAD_SHAPE;
  if (d->num_heads <= 0 || d->num_heads % 16 != 0) return MLA_ERR_BAD_HEADS;
  if (d->page_size != 16 && d->page_size != 32 && d->page_size != 64) return MLA_ERR_BAD_PAGE_SIZE;
  if (d->kv_lora_rank != 512 || d->qk_rope_head_dim != 64) return MLA_ERR_BAD_HEAD_DIMS;
  if (d->kv_dtype != MLA_KV_BF16 && d->kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_BAD_DTYPE;
  if (max_q_len < 1 || d->total_q < 1) return MLA_ERR_BAD_Q_LEN;
  if (!packed && (d->q_len_fixed != max_q_len || (int64_t)d->batch * d->q_len_fixed != d->total_q))
    return MLA_ERR_BAD_Q_LEN;
  if (packed && d->total_q > (int64_t)d->batch * max_q_len) return MLA_ERR_BAD_Q_LEN;
  if ((int64_t)d->block_table_stride * d->page_size < max_seq_len) return MLA_ERR_BAD_BLOCK_TABLE;
  // 32-bit tile arithmetic on device
  const int64_t units = (int64_t)d->batch * ((int64_t)max_q_len * d->num_heads + PAIRS_BLOCK - 1) / PAIRS_BLOCK;
  if (units * ((max_seq_len + TILE - 1) / TILE) >= (int64_t)1 << 30) return MLA_ERR_BAD_SHAPE;
  return MLA_OK;
}

template <bool FP8, int PS>
void launch_decode(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL((mla_decode_kernel<FP8, PS>), dim3(p.grid), dim3(THREADS), 0, s, p);
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MLA_ERR_BAD_HEADS: return "num_heads must be a positive multiple of 16";
    case MLA_ERR_BAD_PAGE_SIZE: return "page_size must be 16, 32 or 64";
    case MLA_ERR_BAD_HEAD_DIMS: return "kv_lora_rank must be 512 and qk_rope_head_dim 64";
    case MLA_ERR_BAD_DTYPE: return "kv_dtype must be bf16 or fp8 e4m3fn";
    case MLA_ERR_MISALIGNED: return "q, kv_cache, out and workspace must be 16-byte aligned";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than mla_decode_paged_workspace_size()";
    case MLA_ERR_BAD_Q_LEN: return "inconsistent query lengths (max_q_len, q_len_fixed, total_q)";
    case MLA_ERR_BAD_BLOCK_TABLE: return "block_table_stride * page_size < max_seq_len";
    case MLA_ERR_BAD_SHAPE: return "batch, max_seq_len or num_pages out of range";
    case MLA_ERR_HIP: return "HIP launch error";
    case MLA_ERR_NO_DEVICE: return "no usable HIP device";
    default: return "unknown status";
  }
}

size_t mla_decode_paged_workspace_size(const mla_decode_dims_t* dims, int32_t max_seq_len, int32_t max_q_len,
                                       int want_lse) {
  (void)want_lse;
  if (dims == nullptr) return 0;
  if (validate(dims, max_seq_len, max_q_len, true) != MLA_OK) return 0;
  int grid = 0;
  if (device_grid(&grid) != MLA_OK) return 0;
  return workspace_layout(grid).total;
}

int mla_decode_paged(const void* q, const void* kv_cache, const int32_t* block_tables, const int32_t* seq_lens,
                     const int32_t* qo_indptr, int32_t max_seq_len, int32_t max_q_len, float bmm1_scale,
                     float bmm2_scale, int causal, void* out, float* lse, void* workspace, size_t workspace_bytes,
                     const mla_decode_dims_t* dims, void* stream) {
  if (!q || !kv_cache || !block_tables || !seq_lens || !out || !workspace || !dims) return MLA_ERR_NULL_POINTER;
  const int v = validate(dims, max_seq_len, max_q_len, qo_indptr != nullptr);
  if (v != MLA_OK) return v;
  if (((uintptr_t)q | (uintptr_t)kv_cache | (uintptr_t)out | (uintptr_t)workspace) & 15) return MLA_ERR_MISALIGNED;
  if (lse != nullptr && ((uintptr_t)lse & 3)) return MLA_ERR_MISALIGNED;
  int grid = 0;
  const int gs = device_grid(&grid);
  if (gs != MLA_OK) return gs;
  const WsLayout wl = workspace_layout(grid);
  if (workspace_bytes < wl.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

  Params p;
  p.q = (const uint16_t*)q;
  p.kv = (const uint8_t*)kv_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.qo_indptr = qo_indptr;
  p.out = (uint16_t*)out;
  p.lse = lse;
  uint8_t* ws = (uint8_t*)workspace;
  p.ws_plan = (int32_t*)(ws + wl.plan_off);
  p.ws_ml = (float*)(ws + wl.ml_off);
  p.ws_o = (float*)(ws + wl.o_off);
  p.batch = dims->batch;
  p.heads = dims->num_heads;
  p.q_len_fixed = qo_indptr ? max_q_len : dims->q_len_fixed;
  p.total_q = dims->total_q;
  p.bt_stride = dims->block_table_stride;
  p.grid = grid;
  p.scale_log2 = bmm1_scale * LOG2E;
  p.bmm2 = bmm2_scale;
  p.causal = causal ? 1 : 0;

  hipStream_t s = (hipStream_t)stream;
  const bool fp8 = dims->kv_dtype == MLA_KV_FP8_E4M3FN;
  void* ev0 = g_ev_start.load(std::memory_order_relaxed);
  void* ev1 = g_ev_stop.load(std::memory_order_relaxed);
  if (ev0 != nullptr) (void)hipEventRecord((hipEvent_t)ev0, s);
  switch (dims->page_size) {
    case 16: fp8 ? launch_decode<true, 16>(p, s) : launch_decode<false, 16>(p, s); break;
    case 32: fp8 ? launch_decode<true, 32>(p, s) : launch_decode<false, 32>(p, s); break;
    default: fp8 ? launch_decode<true, 64>(p, s) : launch_decode<false, 64>(p, s); break;
  }
  if (ev1 != nullptr) (void)hipEventRecord((hipEvent_t)ev1, s);
  const int items = dims->total_q * dims->num_heads;
  hipLaunchKernelGGL(mla_merge_kernel, dim3((items + 3) / 4), dim3(THREADS), 0, s, p);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

void mla_decode_internal_set_grid_override(int32_t grid) { g_grid_override.store(grid > 0 ? grid : 0); }

void mla_decode_internal_set_kernel_events(void* start_event, void* stop_event) {
  g_ev_start.store(start_event);
  g_ev_stop.store(stop_event);
}

int mla_decode_internal_fp8_to_bf16(const void* in, void* out, int64_t n_groups, void* stream) {
  if (!in || !out) return MLA_ERR_NULL_POINTER;
  if (n_groups <= 0) return MLA_OK;
  if (((uintptr_t)in & 7) || ((uintptr_t)out & 15)) return MLA_ERR_MISALIGNED;
  const int64_t blocks = (n_groups + THREADS - 1) / THREADS;
  hipLaunchKernelGGL(fp8_to_bf16_kernel, dim3((unsigned)blocks), dim3(THREADS), 0, (hipStream_t)stream,
                     (const u32x2*)in, (bf16x8*)out, n_groups);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
