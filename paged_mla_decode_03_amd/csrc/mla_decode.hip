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
// Kernel design (one 4-wave workgroup per compute unit, persistent):
//   * Work plan, on device: every workgroup scans seq_lens / qo_indptr
//     (tiles of 32 KV rows per "unit" = request x block of 128 (row, head)
//     pairs), then owns an equal, contiguous range of a cost space that counts
//     every tile and charges each segment start.  A unit cut by range
//     boundaries is written as partials and merged by a second kernel.  When
//     every request holds the same 2, 4 or 8 units, a group of that many
//     workgroups on one XCD walks each range together, one unit each, so a KV
//     tile leaves HBM once per group and its other reads hit L2.  No
//     device-to-host read anywhere.
//   * QK^T: wave w owns 32 pairs with all 576 query dims in VGPRs (MFMA B
//     operand) and computes S^T[32 tokens x 32 pairs] on
//     v_mfma_f32_32x32x16_bf16 with the KV tile as the A operand (rows permuted
//     so the result lands in the layout P.V needs).  The loop runs one tile
//     ahead: the next tile's QK^T MFMAs carry the current tile's softmax
//     between them.
//   * P.V: waves 2g and 2g+1 exchange their bf16 P through LDS; each then
//     accumulates both waves' 64 pairs over one half of the 512 output dims in
//     AGPRs (O^T += V^T . P^T), so every V^T fragment (ds_read_b64_tr_b16, or
//     ds_read_b64_tr_b8 for fp8) feeds two MFMAs.  A tile crosses HBM once per
//     unit and no logits move between waves.
//   * Loader: each wave streams 8 rows of a tile straight into LDS with
//     global_load_lds_dwordx4; a 4-buffer ring keeps two tiles in flight; rows
//     past seq_len are never loaded and are zero-filled instead, so NaN in
//     unused slots cannot leak.  16-byte chunks are XOR-swizzled by row to keep
//     LDS reads conflict-free.  Page ids come from a block-table window held in
//     VGPRs.
//   * Softmax: exp2 domain (log2 e folded into bmm1), one pair per lane column;
//     logits are taken relative to a per-pair reference max fixed by the first
//     visible tile; a logit beyond it by more than 2^32 restarts the segment with
//     the observed max (never happens for sane inputs; keeps O free of rescales).
//   * fp8 E4M3FN KV: QK^T runs on v_mfma_f32_32x32x64_f8f6f4 straight from the
//     landed fp8 tile, with an fp8 query as given or with a bf16 query split per
//     (row, head) into two E4M3 terms under a power-of-two scale (18 MFMAs per
//     tile, exact within 2^9 of the pair's largest element).  V fragments are
//     widened exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8) for the bf16 P.V, as
//     are the rows of the sparse gather.  Scales only enter through bmm1/bmm2.
//   * Options (mla_decode_paged_ex): device-resident scales, per-head attention
//     sinks (one more softmax term, applied in the merge), a sequence-sharded
//     partial mode (causal limits from global lengths), and a sparse top-k
//     layout in which each query row attends to the cache rows its list names
//     (list entries fetched into LDS two tiles ahead of the rows).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <algorithm>
#include <type_traits>
#include <atomic>
#include <mutex>

#include "mla_decode.h"

namespace {

constexpr int D_QK = 576;
constexpr int D_V = 512;
constexpr int TILE = 32;          // KV rows per LDS tile
constexpr int NBUF = 4;           // ring: tile t+1 resident, t+2/t+3 landing, t in use by P.V
constexpr int THREADS = 256;      // 4 waves, one per SIMD
constexpr int WAVES = THREADS / 64;
constexpr int PAIRS_WAVE = 32;    // (row, head) pairs per wave (MFMA N dimension)
constexpr int PAIRS_BLOCK = WAVES * PAIRS_WAVE;  // 128 pairs per unit
constexpr int QK_STEPS = 36;      // 16-dim MFMA steps over 576 dims (32 latent + 4 RoPE)
constexpr int PV_BLOCKS = 16;     // 32-dim output blocks over 512 dims
constexpr int ROWB_BF16 = D_QK * 2;            // 1152
constexpr int ROWB_FP8 = D_QK;                 // 576
constexpr int TILEB = TILE * ROWB_BF16;        // 36864 bytes per buffer (fp8 tiles use half)
constexpr int MERGE_THREADS = 256;     // merge kernel: one wave per (row, head)
constexpr int PLAN_INTS = MLA_MAX_BATCH + 1;
constexpr int PSLOT_OFF = NBUF * TILEB;        // P exchange: [4 waves][2 KB] bf16 P of a tile
constexpr int PSLOT_BYTES = 2048;
constexpr int FLAGS_OFF = PSLOT_OFF + WAVES * PSLOT_BYTES;  // end-of-segment flags
// Sparse top-k lists: each wave's 8 entries of a tile, in a ring of IDX_SLOTS
// tiles, and one byte per wave and tile slot marking the live rows.
constexpr int IDX_SLOTS = 4;
constexpr int IDX_OFF = FLAGS_OFF + 64;
constexpr int VMASK_OFF = IDX_OFF + IDX_SLOTS * WAVES * 32;
constexpr int LDS_BYTES = VMASK_OFF + IDX_SLOTS * 4;
// The work-plan scan (prologue only) aliases the tile buffers while they are idle.
constexpr int PLAN_SCRATCH_OFF = 0;
constexpr int UNIT_SCRATCH_OFF = PLAN_INTS * 4 + 60;
constexpr int SCAN_SCRATCH_OFF = UNIT_SCRATCH_OFF + PLAN_INTS * 4 + 60;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// A segment is redone with a raised reference max only when a logit beats the
// reference by more than 2^32: P and the fp32 sums stay far from overflow below.
constexpr float RESCALE_THRESHOLD = 32.0f;
// Work-split cost of a segment's start (query load, first tiles, O store) in
// tile-equivalents; the split balances tiles plus this per segment.  The
// sparse layout's units are short (a list of K entries), and there a lower
// charge, i.e. more workgroups per unit, measured faster (65.3 against 67.5 us
// for 64 rows x 2048 entries; 2 and 12 were slower).
constexpr int SEG_COST_DEFAULT = 8;
constexpr int SEG_COST_SPARSE = 4;
constexpr int SEG_COST_MAX = 256;

static_assert(LDS_BYTES <= 163840, "LDS budget");
static_assert(IDX_SLOTS == 4, "a segment start fetches four tiles' list entries, one ring slot each");
static_assert(PAIRS_BLOCK * D_V * 2 <= NBUF * TILEB, "the O block is staged in the tile buffers");
static_assert(SCAN_SCRATCH_OFF + 2 * THREADS * 4 <= TILEB, "plan scratch fits in one tile buffer");

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
  uint16_t* ws_o;   // [G + U][128][512] bf16 O per segment (unnormalised)
  float* ws_ml;     // [G + U][128][2]   per segment (max in log2 units, sum)
  int32_t* ws_plan; // [0] = cost per range C, [1] = group size GU (1: none),
                    // [2 + b] = tile offset of request b (b <= B),
                    // [3 + B + b] = first global unit of request b (b <= B)
  int32_t batch;
  int32_t heads;
  int32_t q_len_fixed;
  int32_t total_q;
  int32_t bt_stride;
  int32_t grid;
  float scale_log2;  // bmm1_scale * log2(e)
  float bmm2;
  int32_t causal;
  int32_t seg_cost;  // cost of starting a segment, in tiles (see the work plan)
  int32_t groups;    // nonzero: the plan may group workgroups (see the work plan)
  const float* bmm1_dev;  // device bmm1_scale (replaces scale_log2 / LOG2E) or null
  const float* bmm2_dev;  // device bmm2_scale (replaces bmm2) or null
  const float* sinks;     // device [heads] sink logits (natural log) or null
  const int32_t* seq_lens_global;  // sequence-sharded partial mode: global lengths, or null
  int32_t cp_world;                // ranks sharing each request's rows round-robin
  int32_t cp_rank;                 // this call's rank: local row j is global position j * cp_world + cp_rank
  int32_t sparse_k;                // top-k list length (sparse layout: one query row per request), or 0
};

// Visible local rows of query row qi of a request with q_b rows and L local
// rows.  Causal rows see global positions below Lg - q_b + qi + 1 (Lg = L
// unsharded); with rows shared round-robin, rank r holds the global positions
// r, r + W, ... of which ceil((n - r) / W) lie below n.
__device__ __forceinline__ int visible_rows(const Params& p, int b, int L, int qb, int qi) {
  if (!p.causal) return L;
  if (p.seq_lens_global == nullptr) return L - qb + qi + 1;
  const int n = p.seq_lens_global[b] - qb + qi + 1;
  const int r = p.cp_rank, W = p.cp_world;
  return min(L, n > r ? (n - r + W - 1) / W : 0);
}

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

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane, with
// a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset.  Both bases
// are wave-uniform; readfirstlane pins them to SGPRs even where the call sits
// under a lane-divergent branch.
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

// vmcnt(0) through the builtin, which the compiler's own wait analysis sees:
// registers loaded before it are then known complete, so it inserts no wait
// for them inside the tile loop (where any vmcnt wait would also drain the
// tiles' DMA, which the compiler does not know about).
__device__ __forceinline__ void drain_vector_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// Wait until at most N LDS operations of this wave are outstanding (LDS
// operations complete in issue order, so the older ones are then done).
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" : : "n"(N) : "memory");
}

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

// Max / sum of a value over lanes l and l ^ 32, which hold the two token halves
// of the same pair.  v_permlane32_swap on two copies of the value leaves lane l
// of one copy and lane l ^ 32 of the other in lane l: no LDS round trip.
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 8 E4M3FN bytes -> 8 bf16 (exact: every E4M3FN value is a bf16 value).
// Byte j of (lo, hi) becomes element j.  gfx950's v_cvt_scalef32_pk_bf16_fp8
// widens two codes (bytes 0-1, or 2-3 with the word select) straight to bf16;
// with a scale of 1 it is the plain conversion.  Four instructions per eight
// codes, half of what a detour through f32 costs.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Two floats -> two bf16 (round to nearest even) in one dword, a in the low
// half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// Elements j, j + 1 (j even) of a bf16x8 as one packed word, and the sum of
// the two bf16 values of a packed word in fp32.
__device__ __forceinline__ void put_p(bf16x8& v, int j, uint32_t word) {
  u32x4 w = __builtin_bit_cast(u32x4, v);
  w[j >> 1] = word;
  v = __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ uint32_t get_p(const bf16x8& v, int j) { return __builtin_bit_cast(u32x4, v)[j >> 1]; }
__device__ __forceinline__ float sum_bf16x2(uint32_t word) {
  return __uint_as_float(word << 16) + __uint_as_float(word & 0xffff0000u);
}

// ---------------------------------------------------------------- matrix-core ops
//
// The MFMAs are issued through inline asm so that the register class of each
// accumulator is ours to choose: the 512 output accumulators of a wave live in
// AGPRs, the QK^T accumulator and everything else in VGPRs (with compiler MFMA
// builtins every accumulator of a kernel allowed more than 256 VGPRs lands in
// AGPRs, which does not fit here).  The asm carries the gfx950 wait states the
// compiler would otherwise insert: each MFMA is preceded by s_nop 1 (a VALU
// write of an A/B operand needs two wait states before the MFMA reads it; the
// nop issues while the previous MFMA still occupies the matrix core), and
// mfma_fence() gives the 12 wait states an MFMA result needs before any other
// instruction reads it.  Back-to-back MFMAs that accumulate into the same
// registers need none.
//
// NOP = false drops the leading s_nop where no operand is written by a VALU
// instruction (bf16 cache: every A/B operand comes from LDS or was written
// long before); the emitted assembly is checked for the wait-state rules in
// the CPU tests.  With an fp8 cache the operands are widened by VALU
// instructions just before, and the s_nop stays.
template <bool NOP = true>
__device__ __forceinline__ void mfma_acc_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (NOP) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <bool NOP = true>
__device__ __forceinline__ void mfma_acc_vgpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (NOP) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
template <bool NOP = true>
__device__ __forceinline__ f32x16 mfma_first_vgpr(const bf16x8& a, const bf16x8& b) {
  f32x16 d;
  if constexpr (NOP) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma_fence(f32x16& v) { asm volatile("s_nop 7\n\ts_nop 3" : "+v"(v)); }

// The fp8 query path's QK^T: v_mfma_f32_32x32x64_f8f6f4 with both operands
// OCP E4M3 (format fields 0), fp32 accumulation, 16 passes.  Its result needs
// 20 wait states before any other instruction reads it (what the compiler
// emits for the builtin), hence mfma8_fence().
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void mfma8_acc_vgpr(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ f32x16 mfma8_first_vgpr(const i32x8& a, const i32x8& b) {
  f32x16 d;
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma8_fence(f32x16& v) { asm volatile("s_nop 15\n\ts_nop 3" : "+v"(v)); }

// ---------------------------------------------------------------- tile layout
//
// One LDS tile buffer holds 32 cache rows split in two blocks:
//   bf16: latent block [32][1024 B] at 0, RoPE block [32][128 B] at 32768;
//   fp8 : latent block [32][512 B]  at 0, RoPE block [32][64 B]  at 16384.
// A latent row is then one 64-lane x 16 B load (bf16) or half of one (fp8).
// 16-byte chunks are XOR-swizzled by row so that both operand reads are
// bank-conflict free:
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
  // zeros made in place (a zero vector kept live across the loop only gets spilled)
  uint32_t z0, z1, z2, z3;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
  asm volatile("v_mov_b32 %0, 0" : "=v"(z1));
  asm volatile("v_mov_b32 %0, 0" : "=v"(z2));
  asm volatile("v_mov_b32 %0, 0" : "=v"(z3));
  *(__attribute__((address_space(3))) u32x4*)((__attribute__((address_space(3))) uint8_t*)smem + off) =
      u32x4{z0, z1, z2, z3};
}

// ---------------------------------------------------------------- work plan

// tile_off[b] = first cost-space tile of request b, tile_off[B] = total tiles;
// unit_off[b] = first cost unit of request b, unit_off[B] = total cost units.
// A request contributes ceil(q_b*H / 128) units of ceil(L_b / 32) tiles each.
// When every request has the same U units, U is 2, 4 or 8, U divides the
// workgroups of each XCD and groups are allowed, the plan groups workgroups
// (return value U): a request is then a single cost unit of ceil(L_b / 32)
// tiles whose units the U workgroups of a group share out.  Otherwise it
// returns 1 and each unit is a cost unit.  Every workgroup reaches the same
// decision from the same lengths.
// 128-pair units and 32-row tiles of request b (lengths outside the documented
// ranges count as empty, so that the work walk always advances)
__device__ __forceinline__ int request_units(const Params& p, int qb) { return max(0, ceil_div(qb * p.heads, PAIRS_BLOCK)); }
// Rows of request b: its length, or the top-k list length in the sparse
// layout (where every query row is a request of its own).
__device__ __forceinline__ int req_len(const Params& p, int b) { return p.sparse_k > 0 ? p.sparse_k : p.seq_lens[b]; }
__device__ __forceinline__ int request_tiles(const Params& p, int b) { return max(0, ceil_div(req_len(p, b), TILE)); }

__device__ int build_plan(const Params& p, int* tile_off, int* unit_off, int* scan) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int B = p.batch;
  constexpr int PER_MAX = (MLA_MAX_BATCH + THREADS - 1) / THREADS;
  const int per = (B + THREADS - 1) / THREADS;
  const int b0 = min(B, tid * per);
  // this thread's requests, kept in registers for the second pass
  int t_b[PER_MAX], u_b[PER_MAX];
  // sums over this thread's requests for both layouts (unit by unit, and one
  // cost unit per request), and the range of unit counts
  int tiles = 0, units = 0, rtiles = 0, rcount = 0, umin = 0x7fffffff, umax = 0;
#pragma unroll
  for (int i = 0; i < PER_MAX; ++i) {
    int t = 0, u = 0;
    if (i < per && b0 + i < B) {
      int r0;
      u = request_units(p, request_rows(p, b0 + i, r0));
      t = request_tiles(p, b0 + i);
      umin = min(umin, u);
      umax = max(umax, u);
    }
    t_b[i] = t;
    u_b[i] = u;
    tiles += u * t;
    units += u;
    rtiles += u > 0 ? t : 0;
    rcount += u > 0 ? 1 : 0;
  }
  // inclusive prefix sums: within each wave by shuffles, then the four wave
  // totals through LDS (one barrier); the unit-count range rides along
  int v[4] = {tiles, units, rtiles, rcount};
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int x = __shfl_up(v[k], off, 64);
      if (lane >= off) v[k] += x;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    umin = min(umin, __shfl_xor(umin, off, 64));
    umax = max(umax, __shfl_xor(umax, off, 64));
  }
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < 4; ++k) scan[k * WAVES + w] = v[k];
    scan[4 * WAVES + w] = umin;
    scan[5 * WAVES + w] = umax;
  }
  __syncthreads();
  int base[4] = {0, 0, 0, 0}, total[4] = {0, 0, 0, 0};
  int gmin = 0x7fffffff, gmax = 0;
  for (int k2 = 0; k2 < WAVES; ++k2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k2 < w) base[k] += scan[k * WAVES + k2];
      total[k] += scan[k * WAVES + k2];
    }
    gmin = min(gmin, scan[4 * WAVES + k2]);
    gmax = max(gmax, scan[5 * WAVES + k2]);
  }
  const int U = gmax;
  const int GU = (p.groups != 0 && gmin == gmax && (U == 2 || U == 4 || U == 8) && p.grid % (8 * U) == 0) ? U : 1;
  const bool grouped = GU > 1;
  int run_t = base[grouped ? 2 : 0] + v[grouped ? 2 : 0] - (grouped ? rtiles : tiles);
  int run_u = base[grouped ? 3 : 1] + v[grouped ? 3 : 1] - (grouped ? rcount : units);
#pragma unroll
  for (int i = 0; i < PER_MAX; ++i) {
    if (i < per && b0 + i < B) {
      tile_off[b0 + i] = run_t;
      unit_off[b0 + i] = run_u;
    }
    const int uc = grouped ? min(u_b[i], 1) : u_b[i];
    run_t += uc * t_b[i];
    run_u += uc;
  }
  if (tid == THREADS - 1) {
    tile_off[B] = total[grouped ? 2 : 0];
    unit_off[B] = total[grouped ? 3 : 1];
  }
  __syncthreads();
  return GU;
}

// ---------------------------------------------------------------- page-id window
//
// A segment's block-table entries are read once, WIN (128 or 64) at a time,
// into one or two VGPRs (lane i holds entries base + i and base + 64 + i); each
// tile's page id is then a v_readlane, so issuing a tile's loads never waits on
// memory.  The fp8 kernels keep a 64-entry window: their tile loop has no
// register to spare for the second one.
struct PageWin {
  int base;  // first block-table index held (wave-uniform)
  int lo;    // entry base + lane
  int hi;    // entry base + 64 + lane
};

// Entries past the request's last page are never read (they may be garbage).
template <int WIN>
__device__ __forceinline__ void load_page_window(const Params& p, int b, int npages, int base, PageWin& pw) {
  const int lane = threadIdx.x & 63;
  const int32_t* row = p.block_tables + (size_t)b * p.bt_stride;
  pw.base = base;
  pw.lo = (base + lane < npages) ? row[base + lane] : 0;
  pw.hi = (WIN > 64 && base + 64 + lane < npages) ? row[base + 64 + lane] : 0;
  drain_vector_loads();
}

// ---------------------------------------------------------------- tile loader

// Page id of cache row `row` (< L) of request b, from the window (refilled when
// the row's page lies past it: drain the loads in flight so the refill is the
// only vector load the following waits can see, then read the next WIN).
template <int PS, int WIN>
__device__ __forceinline__ int page_id(const Params& p, int b, int L, int row, PageWin& pw) {
  int pi = uniform(row / PS - pw.base);
  if (pi >= WIN) {
    wait_vmcnt<0>();
    load_page_window<WIN>(p, b, ceil_div(L, PS), row / PS, pw);
    pi = 0;
  }
  if (WIN <= 64) return uniform(__builtin_amdgcn_readlane(pw.lo, pi));
  return uniform(pi < 64 ? __builtin_amdgcn_readlane(pw.lo, pi) : __builtin_amdgcn_readlane(pw.hi, pi - 64));
}

template <bool FP8>
constexpr int page_window() { return FP8 ? 64 : 128; }

// DMA instructions one wave issues for a full tile.
template <bool FP8>
constexpr int tile_loads() { return FP8 ? 5 : 9; }

// A wave's share of one tile load: rows [8w, 8w+8) of tile t, which always sit
// in one page (page_size is a multiple of 16), so the page base is wave-uniform.
// prepare_tile() does everything except the DMA of a full 8-row share: rows at
// or past seq_len are never read from memory (nor is their block-table entry)
// and are zero-filled; a share cut by seq_len is loaded at once.  A full share
// is returned for issue_tile_share(), so that the caller picks the moment: a
// burst of DMA instructions stalls the issuing wave while the CU's address
// unit works through them, and bursts from several waves queue behind each
// other.
struct TileLoad {
  const uint8_t* pg;  // global address of the share's first row; null: nothing left to issue
  uint32_t lat;       // LDS byte address of the share's first latent row
  uint32_t rope;      // LDS byte address of the share's RoPE rows
};

template <bool FP8, int PS>
__device__ __forceinline__ TileLoad prepare_tile(const Params& p, uint8_t* smem, uint32_t buf, int b, int L, int t,
                                                 PageWin& pw) {
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int row0 = t * TILE + 8 * w;
  const uint32_t lds0 = lds_addr(smem);
  TileLoad tl{nullptr, 0u, 0u};
  {
    // the common case in straight-line scalar code: a full share whose page id
    // is in the window
    constexpr int WIN = page_window<FP8>();
    const int pi = uniform(row0 / PS - pw.base);
    if (row0 + 8 <= L && pi < WIN) {
      const int e_lo = __builtin_amdgcn_readlane(pw.lo, pi & 63);
      const int e_hi = (WIN > 64) ? __builtin_amdgcn_readlane(pw.hi, pi & 63) : e_lo;
      const int page = uniform(pi < 64 ? e_lo : e_hi);
      const size_t rowb = FP8 ? ROWB_FP8 : ROWB_BF16;
      const uint8_t* pg = p.kv + ((size_t)page * PS + (row0 % PS)) * rowb;
      if (!FP8) return TileLoad{pg, lds0 + buf + 8 * w * 1024, lds0 + buf + ROPE_OFF_BF16 + 8 * w * 128};
      return TileLoad{pg, lds0 + buf + 8 * w * 512, lds0 + buf + ROPE_OFF_FP8 + 8 * w * 64};
    }
  }
  if (!FP8) {
    const uint32_t lat = buf + 8 * w * 1024;
    const uint32_t rope = buf + ROPE_OFF_BF16 + 8 * w * 128;
    if (row0 >= L) {
#pragma unroll
      for (int i = 0; i < 8; ++i) lds_zero16(smem, lat + i * 1024 + lane * 16);
      lds_zero16(smem, rope + lane * 16);
      return tl;
    }
    const int page = page_id<PS, page_window<FP8>()>(p, b, L, row0, pw);
    const uint8_t* pg = p.kv + ((size_t)page * PS + (row0 % PS)) * ROWB_BF16;
    const int nvalid = L - row0;
    if (nvalid >= 8) return TileLoad{pg, lds0 + lat, lds0 + rope};
    // swizzles use the row's place in the tile (8w + i)
    const int rr = lane >> 3;  // RoPE: 8 lanes per row
    const uint32_t rope_off = (uint32_t)(rr * ROWB_BF16 + 1024 + (((lane & 7) ^ swz_rope_bf16(8 * w + rr)) << 4));
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
      return tl;
    }
    const int page = page_id<PS, page_window<FP8>()>(p, b, L, row0, pw);
    const uint8_t* pg = p.kv + ((size_t)page * PS + (row0 % PS)) * ROWB_FP8;
    const int nvalid = L - row0;
    if (nvalid >= 8) return TileLoad{pg, lds0 + lat, lds0 + rope};
    const int hi = lane >> 5;
    const int rr = lane >> 2;  // RoPE: 4 lanes per row, 32 lanes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 2 * i + hi;
      if (r < nvalid)
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
  return tl;
}

// Four DMA instructions with one m0: the instruction offsets 0, 1024, 2048 and
// 3072 step the LDS destination m0 + offset + 16 * lane and the global address
// sbase + voff + offset together, so rows whose global stride differs from
// their 1 KiB LDS stride carry the difference in their lane offsets.  Writing
// m0 costs the issuing wave about ten cycles per LDS-DMA instruction that
// follows it, so it is written once per four instructions.
__device__ __forceinline__ void dma16x4_s(const void* sbase, uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                          uint32_t lds_wave_base) {
  const uint64_t sb = (uint64_t)(uintptr_t)sbase;
  const uint64_t sbu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32)) << 32);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile(
      "s_mov_b32 m0, %5\n\t"
      "global_load_lds_dwordx4 %0, %4\n\t"
      "global_load_lds_dwordx4 %1, %4 offset:1024\n\t"
      "global_load_lds_dwordx4 %2, %4 offset:2048\n\t"
      "global_load_lds_dwordx4 %3, %4 offset:3072"
      :
      : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"((const void*)(uintptr_t)sbu), "s"(m0)
      : "memory");
}

// The DMA instructions of a full share (tile_loads<FP8>() of them, in a fixed
// order); nothing for an empty share.
template <bool FP8>
__device__ __forceinline__ void issue_tile_share(const TileLoad& tl) {
  if (tl.pg == nullptr) return;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  if (!FP8) {
    // latent row i: global pg + 1152 i + 16 (lane ^ swz), LDS lat + 1024 i + 16 lane
    auto voff = [&](int i) { return (uint32_t)(((lane ^ swz_lat_bf16(8 * w + i)) << 4) + 128 * (i & 3)); };
    dma16x4_s(tl.pg, voff(0), voff(1), voff(2), voff(3), tl.lat);
    dma16x4_s(tl.pg + 4 * ROWB_BF16, voff(4), voff(5), voff(6), voff(7), tl.lat + 4096);
    const int rr = lane >> 3;
    dma16_s(tl.pg, (uint32_t)(rr * ROWB_BF16 + 1024 + (((lane & 7) ^ swz_rope_bf16(8 * w + rr)) << 4)), tl.rope);
  } else {
    // latent rows 2k, 2k+1 (lane halves): global pg + 1152 k + 576 hi, LDS lat + 1024 k
    const int hi = lane >> 5;
    auto voff = [&](int k) {
      return (uint32_t)(hi * ROWB_FP8 + (((lane & 31) ^ swz_lat_fp8(8 * w + 2 * k + hi)) << 4) + 128 * k);
    };
    dma16x4_s(tl.pg, voff(0), voff(1), voff(2), voff(3), tl.lat);
    if (lane < 32) {
      const int rr = lane >> 2;
      dma16_s(tl.pg, (uint32_t)(rr * ROWB_FP8 + 512 + (((lane & 3) ^ swz_rope_fp8(8 * w + rr)) << 4)), tl.rope);
    }
  }
}

// A whole tile load at once.  A full tile costs each wave exactly
// tile_loads<FP8>() DMA instructions.
template <bool FP8, int PS>
__device__ __forceinline__ void issue_tile(const Params& p, uint8_t* smem, uint32_t buf, int b, int L, int t,
                                           PageWin& pw) {
  issue_tile_share<FP8>(prepare_tile<FP8, PS>(p, smem, buf, b, L, t, pw));
}

// ---------------------------------------------------------------- sparse top-k gather
//
// In the sparse layout (FlashInfer's sparse_mla_top_k; the list layout is this
// library's reading) a unit is one query row and its tile t holds entries
// 32t .. 32t + 31 of the row's list: entry e >= 0 is cache row e, at
// kv + e * row bytes (the pages are contiguous, so that is page e / page_size,
// slot e % page_size); a negative entry, or a position past top-k, is an empty
// row.  A wave's share of a tile (rows 8w .. 8w + 7) needs its 8 entries
// before its DMA can be issued: one 4-byte-per-lane LDS DMA fetches them into
// a ring two tiles ahead, in the same vmcnt stream as the tiles.  Every share
// issues the same instructions (an empty row's with no lanes, its LDS row
// zero-filled) and publishes one byte of live-row bits for the softmax.

// One DMA instruction of 4 bytes per lane (wave-uniform base + lane offset)
// under a lane mask.  With no lanes it still issues and counts in vmcnt; exec
// is restored inside the asm, and the s_nop covers the wait states an exec
// write owes later lane-crossing VALU instructions.
__device__ __forceinline__ void dma4_m(const void* sbase, uint32_t voff, uint32_t lds_wave_base, uint64_t lanes) {
  const uint64_t sb = (uint64_t)(uintptr_t)sbase;
  const uint64_t sbu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32)) << 32);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)lanes);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(lanes >> 32));
  uint64_t save;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_and_b32 exec_lo, exec_lo, %4\n\t"
      "s_and_b32 exec_hi, exec_hi, %5\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b64 exec, %0\n\t"
      "s_nop 4"
      : "=&s"(save)
      : "v"(voff), "s"((const void*)(uintptr_t)sbu), "s"(m0), "s"(lo), "s"(hi)
      : "memory");
}

// One 16-byte-per-lane DMA instruction from per-lane 64-bit addresses under a
// lane mask (rows of a share sit anywhere in the cache).
__device__ __forceinline__ void dma16_vm(uint64_t vaddr, uint32_t lds_wave_base, uint64_t lanes) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)lanes);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(lanes >> 32));
  uint64_t save;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_and_b32 exec_lo, exec_lo, %3\n\t"
      "s_and_b32 exec_hi, exec_hi, %4\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b64 exec, %0\n\t"
      "s_nop 4"
      : "=&s"(save)
      : "v"(vaddr), "s"(m0), "s"(lo), "s"(hi)
      : "memory");
}

__device__ __forceinline__ uint32_t idx_slot_off(int t, int w) {
  return IDX_OFF + (uint32_t)(t & (IDX_SLOTS - 1)) * (WAVES * 32) + (uint32_t)w * 32;
}

// Fetch the list entries of this wave's share of tile t (lanes 0..7; none
// when !live or past top-k): exactly one instruction.
__device__ __forceinline__ void issue_sparse_index(const Params& p, uint8_t* smem, int b, int t, bool live) {
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int j0 = live ? t * TILE + 8 * w : 0;
  const int32_t* lst = p.block_tables + (size_t)b * p.bt_stride + j0;
  const uint64_t lanes = __builtin_amdgcn_ballot_w64(live && lane < 8 && j0 + lane < p.sparse_k);
  dma4_m(lst, (uint32_t)lane * 4, lds_addr(smem) + idx_slot_off(t, w), lanes);
}

// The DMA of this wave's share of tile t into buffer buf (its entries have
// landed): tile_loads<FP8>() instructions, empty rows zero-filled.
template <bool FP8>
__device__ __forceinline__ void issue_sparse_share(const Params& p, uint8_t* smem, uint32_t buf, int t) {
  // (the empty asm makes the lane id opaque, so the per-lane offsets below are
  // recomputed at each call instead of being hoisted into registers that would
  // stay live across the whole tile loop)
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int w = uniform(threadIdx.x >> 6);
  const int j0 = t * TILE + 8 * w;
  const uint32_t lds0 = lds_addr(smem);
  auto pick = [&](int r) {  // entry r of the share (lane-varying r), read from the ring
    const int v = *(const __attribute__((address_space(3))) int*)((const __attribute__((address_space(3))) uint8_t*)smem +
                                                                 idx_slot_off(t, w) + 4 * r);
    return (j0 + r < p.sparse_k) ? v : -1;  // positions past top-k hold stale ring data
  };
  const int mine = pick(lane & 7);  // lane i < 8: entry i
  const uint32_t live8 = (uint32_t)__builtin_amdgcn_ballot_w64(lane < 8 && mine >= 0) & 0xFFu;
  if (lane == 0)
    *((__attribute__((address_space(3))) uint8_t*)smem + VMASK_OFF + (t & (IDX_SLOTS - 1)) * 4 + w) = (uint8_t)live8;
  const uint64_t kv = (uint64_t)(uintptr_t)p.kv;
  if (!FP8) {
    const uint32_t lat = buf + 8 * w * 1024;
    const uint32_t rope = buf + ROPE_OFF_BF16 + 8 * w * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ei = uniform(__builtin_amdgcn_readlane(mine, i));
      if (ei < 0) lds_zero16(smem, lat + i * 1024 + lane * 16);
      const uint64_t a = kv + (uint64_t)max(ei, 0) * ROWB_BF16 + (uint32_t)((lane ^ swz_lat_bf16(8 * w + i)) << 4);
      dma16_vm(a, lds0 + lat + i * 1024, ei >= 0 ? ~0ull : 0ull);
    }
    const int rr = lane >> 3;  // RoPE: 8 lanes per row
    const int er = pick(rr);
    if (er < 0) lds_zero16(smem, rope + lane * 16);
    const uint64_t a = kv + (uint64_t)max(er, 0) * ROWB_BF16 + 1024 +
                       (uint32_t)((((lane & 7) ^ swz_rope_bf16(8 * w + rr))) << 4);
    dma16_vm(a, lds0 + rope, __builtin_amdgcn_ballot_w64(er >= 0));
  } else {
    const uint32_t lat = buf + 8 * w * 512;
    const uint32_t rope = buf + ROPE_OFF_FP8 + 8 * w * 64;
    const int hi = lane >> 5;  // latent: rows 2k (lanes 0..31) and 2k + 1 (lanes 32..63)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 2 * k + hi;
      const int er = pick(r);
      if (er < 0) lds_zero16(smem, lat + k * 1024 + lane * 16);
      const uint64_t a = kv + (uint64_t)max(er, 0) * ROWB_FP8 + (uint32_t)(((lane & 31) ^ swz_lat_fp8(8 * w + r)) << 4);
      dma16_vm(a, lds0 + lat + k * 1024, __builtin_amdgcn_ballot_w64(er >= 0));
    }
    const int rr = (lane & 31) >> 2;  // RoPE: 4 lanes per row, lanes 0..31
    const int er = pick(rr);
    if (lane < 32 && er < 0) lds_zero16(smem, rope + lane * 16);
    const uint64_t a = kv + (uint64_t)max(er, 0) * ROWB_FP8 + 512 + (uint32_t)(((lane & 3) ^ swz_rope_fp8(8 * w + rr)) << 4);
    dma16_vm(a, lds0 + rope, __builtin_amdgcn_ballot_w64(lane < 32 && er >= 0));
  }
}

// ---------------------------------------------------------------- one segment
//
// A unit is (request, block of 128 (row, head) pairs); wave w owns pairs
// [32w, 32w+32) of it with the full 576-dim query and the full 512-dim output.
//
// Software pipeline over tiles (4 LDS buffers), iteration t:
//   wait + barrier -> tile t+1 is in LDS, tile t-1's buffer is free: issue tile t+3
//   QK^T(t+1) on the matrix cores, softmax(t) on the VALU alongside
//   P.V(t)
// Waves with no pairs run the same barrier and DMA sequence only.

// Per-lane state of an active wave.
struct SegState {
  f32x16 acc[PV_BLOCKS];  // O^T accumulators: [2d] own pairs, [2d + 1] the partner's; dim block d of the half
  float m_ref;     // reference max, log2 units (identical in both lane halves)
  float m_max;     // largest logit of the masked-path tiles, log2 units (both halves)
  float s_max;     // largest raw score of the fast-path tiles (this lane's tokens only)
  float lsum;      // this lane's share of the softmax denominator
  bool ref_ready;  // wave-uniform: every lane's m_ref is set
};

// Query modes (QM): 0 = bf16 query on the bf16 MFMA (fp8 cache rows widened);
// 1 = fp8 query codes on the fp8 MFMA; 2 = bf16 query split into two fp8 terms
// (q 2^e = q_hi + q_lo) on the fp8 MFMA, for an fp8 cache.  c is the logit
// scale in log2 units of the lane's scores (mode 2: divided by 2^e).
// OWN / PARTNER: some pair of this wave's / the partner's 32 QK^T pairs
// exists.  In an active group the even wave's pairs always do; when the odd
// wave's do not (a unit of at most 32, or 65 to 96, pairs), the odd wave skips
// its QK^T and softmax and both waves skip the P.V MFMAs of those pairs, whose
// results would be discarded.
template <bool FP8, int PS, bool ACTIVE, int QM, bool OWN, bool PARTNER, typename QF>
__device__ __forceinline__ void segment_loop(const Params& p, uint8_t* smem, int b, int L, int t0, int t1,
                                             const QF& qf, float c, int n_vis, int min_vis,
                                             SegState& st, PageWin& pw) {
  static_assert(!ACTIVE || OWN || PARTNER, "an active group has live pairs");
  constexpr bool Q8 = QM != 0;
  constexpr int LOADS = tile_loads<FP8>();
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
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
  uint32_t qa_lat, qa_rope, tr_base;
  int qs_lat, qs_rope, tr_sl, tr_cc, tr_z;
  if (!FP8) {
    const int sl = swz_lat_bf16(prow);
    qa_lat = prow * 1024 + 16 * (h ^ (sl & 1));
    qs_lat = sl >> 1;
    qa_rope = ROPE_OFF_BF16 + prow * 128;
    qs_rope = swz_rope_bf16(prow);
    tr_sl = s16 >> 2;
    tr_cc = 2 * g1 + ((s16 & 3) >> 1);
    tr_base = (8 * h + tr_sl) * 1024 + 8 * (s16 & 1);
    tr_z = 0;
  } else {
    qa_lat = prow * 512 + 8 * h;
    qs_lat = swz_lat_fp8(prow);
    qa_rope = ROPE_OFF_FP8 + prow * 64 + 8 * h;
    qs_rope = swz_rope_fp8(prow);
    tr_z = s16 >> 1;
    tr_base = (8 * h + tr_z) * 512 + 8 * (s16 & 1);
    tr_sl = tr_cc = 0;
  }

  // Per-buffer bases: every per-step offset below is the base XORed with a
  // step constant (the lane-dependent swizzle bits sit in bits that the buffer
  // offset and the tile rows never touch) plus an instruction immediate, so a
  // wave keeps a few base registers instead of one address per step.
  //   bf16 A : base | 32 qs (bits 5..7), step kk: ^ 32(kk&7), + 256(kk>>3)
  //   bf16 V : base | 64 tr_sl | 16 (tr_cc ^ 2h) (bits 4..7) + 512 dh, block d of the
  //            half, chunk c: ^ 64(d&3), + 256(d>>2) + 16384c; second half-read ^ 16, + 4096
  //   fp8  A : base | 16 qs (bits 4..7), step kk: ^ 16 kk
  //   fp8  V : base | 16 (g1 ^ (8h + tr_z)) (bits 4..7) + 256 dh, block d: ^ 32 d, + 8192c
  const uint32_t a_lane = FP8 ? qa_lat + 16 * qs_lat : qa_lat + 32 * qs_lat;
  const uint32_t ps_own = PSLOT_OFF + w * PSLOT_BYTES + lane * 16;
  const uint32_t ps_other = PSLOT_OFF + (w ^ 1) * PSLOT_BYTES + lane * 16;
  const int dh = w & 1;  // P.V output half: dims [256 dh, 256 dh + 256)
  const uint32_t v_lane = FP8 ? tr_base + 16 * (g1 ^ (8 * h + tr_z)) + 256 * dh
                              : tr_base + 64 * tr_sl + 16 * (tr_cc ^ (2 * h)) + 512 * dh;
  // (the empty asm keeps the compiler from folding a known buffer offset into
  // per-step lane constants that would then stay live across the whole kernel)
  auto opaque = [](uint32_t v) -> uint32_t {
    asm volatile("" : "+v"(v));
    return v;
  };
  // A fragment for 16-dim step kk (0..31 latent, 32..35 RoPE)
  auto load_a = [&](uint32_t buf, int kk) -> u32x4 {
    if (FP8) {
      const uint32_t off = (kk < 32) ? ((buf + a_lane) ^ (16u * (kk & 15))) + 256 * (kk >> 4)
                                     : buf + qa_rope + 16 * ((kk - 32) ^ qs_rope);
      const u32x2 raw = lds_read_b64(smem, off);
      return u32x4{raw[0], raw[1], 0u, 0u};
    } else {
      const uint32_t off = (kk < 32) ? ((buf + a_lane) ^ (32u * (kk & 7))) + 256 * (kk >> 3)
                                     : buf + qa_rope + 16 * ((2 * (kk - 32) + h) ^ qs_rope);
      return lds_read_b128(smem, off);
    }
  };
  // V^T fragment for step = c * 8 + d (chunk c of 16 tokens, dim block d of 32 in this
  // wave's output half)
  auto load_v = [&](uint32_t buf, int step) -> u32x4 {
    const int c = step >> 3, d = step & 7;
    if (FP8) {
      const uint32_t off = ((buf + v_lane) ^ (32u * d)) + 16 * c * 512;
      const i32x2 raw = lds_read_tr8(smem, off);
      return u32x4{(uint32_t)raw[0], (uint32_t)raw[1], 0u, 0u};
    } else {
      const uint32_t base = ((buf + v_lane) ^ (64u * (d & 3))) + 16 * c * 1024 + 256 * (d >> 2);
      const s16x4 lo = lds_read_tr16(smem, base);
      const s16x4 hi = lds_read_tr16(smem, (base ^ 16u) + 4 * 1024);
      return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto to_bf16 = [&](const u32x4& raw) -> bf16x8 {
    return FP8 ? fp8x8_to_bf16x8(raw[0], raw[1]) : __builtin_bit_cast(bf16x8, raw);
  };
  // QK^T of the tile in buf.  fill(k) runs right after MFMA k: independent VALU
  // work (the previous tile's softmax) that the wave issues while the matrix
  // core is busy; the scheduling barrier keeps each piece in its slot.  pre()
  // runs once the first A fragments are requested, before the first MFMA.
  // fp8 query: A fragment of 64-dim step kk (0..7 latent, 8 RoPE) is 32 bytes
  // of the lane's row, chunks 4kk + 2h and 4kk + 2h + 1 (RoPE: 2h, 2h + 1), the
  // same bytes the lane's query fragment holds, so the MFMA pairs them
  // whatever its internal order of the 64 products.
  const int s8 = swz_lat_fp8(prow);
  const int s8r = swz_rope_fp8(prow);
  auto load_a8 = [&](uint32_t buf, int kk) -> i32x8 {
    uint32_t o0, o1;
    if (kk < 8) {
      o0 = buf + prow * 512 + ((16u * ((2 * h) ^ s8)) ^ (64u * kk));
      o1 = buf + prow * 512 + ((16u * ((2 * h + 1) ^ s8)) ^ (64u * kk));
    } else {
      o0 = buf + ROPE_OFF_FP8 + prow * 64 + 16 * ((2 * h) ^ s8r);
      o1 = buf + ROPE_OFF_FP8 + prow * 64 + 16 * ((2 * h + 1) ^ s8r);
    }
    const u32x4 x = lds_read_b128(smem, o0);
    const u32x4 y = lds_read_b128(smem, o1);
    return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
  };
  auto qk = [&](uint32_t buf_in, auto&& fill, auto&& pre) -> f32x16 {
    const uint32_t buf = opaque(buf_in);
    f32x16 s;
    if constexpr (Q8) {
      // 9 MFMAs of 64 dims (split query: 9 pairs, high term then low term);
      // fill() gets two slots per step (0..17)
      constexpr int GA8 = 2;  // A fragments read this many steps ahead
      i32x8 araw8[GA8];
#pragma unroll
      for (int k = 0; k < GA8; ++k) araw8[k] = load_a8(buf, k);
      pre();
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const i32x8 cur = araw8[k % GA8];
        if (k + GA8 < 9) araw8[k % GA8] = load_a8(buf, k + GA8);
        if (k == 0) s = mfma8_first_vgpr(cur, qf[0]);
        else mfma8_acc_vgpr(s, cur, qf[k]);
        fill(2 * k);
        if constexpr (QM == 2) {
          // the low term of the split query, back to back on the same accumulator
          __builtin_amdgcn_sched_barrier(0);
          mfma8_acc_vgpr(s, cur, qf[9 + k]);
        }
        fill(2 * k + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma8_fence(s);
      return s;
    } else {
      constexpr int GA = 4;  // A fragments read this many steps ahead
      u32x4 araw[GA];
#pragma unroll
      for (int k = 0; k < GA; ++k) araw[k] = load_a(buf, k);
      pre();
#pragma unroll
      for (int k = 0; k < QK_STEPS; ++k) {
        const u32x4 cur = araw[k % GA];
        if (k + GA < QK_STEPS) araw[k % GA] = load_a(buf, k + GA);
        if (k == 0) s = mfma_first_vgpr<FP8>(to_bf16(cur), qf[k]);
        else mfma_acc_vgpr<FP8>(s, to_bf16(cur), qf[k]);
        fill(k);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_fence(s);
      return s;
    }
  };
  static_assert(!Q8 || FP8, "an fp8 query needs the fp8 cache");
  auto no_fill = [](int) {};
  auto no_pre = [] {};

  // Tile t has landed once at most the DMA ops of the n tiles issued after it
  // remain; a partial tile among them makes the count unknown, so drain.
  // (Sparse layout: each tile's DMA is followed by the list fetch of the tile
  // two further on, so the same wait also lands the entries the next share
  // issue reads.)
  constexpr int PER_TILE = LOADS + (PS == 0 ? 1 : 0);
  auto wait_tile = [&](int t, int n) {
    n = min(n, t1 - 1 - t);
    if (n <= 0 || (t + n + 1) * TILE > L) wait_vmcnt<0>();
    else if (n == 1) wait_vmcnt<PER_TILE>();
    else wait_vmcnt<2 * PER_TILE>();
  };

  // the fast path needs logits increasing with the raw scores; c has the
  // sign of bmm1 in every lane (split mode keeps it from underflowing), so
  // this test is wave-uniform
  const bool c_pos = c > 0.f;

  // ---------------- softmax (exp2 domain) of one tile's scores s; value k is
  // token 16(k>>3) + 8h + (k&7) of the tile.
  // Fast path (every token of the tile visible to every pair of this wave, the
  // reference fixed): the exponentials depend on nothing but the scores, and
  // the running max only feeds the overflow check at the segment's end.  It is
  // cut into QK_STEPS pieces so that it can sit between the next tile's MFMAs.
  // Pieces 4m .. 4m+3 handle tokens j, j+1 of both lane halves' 8-token runs
  // (j = 2m): two exponentials, two more, the bf16 packing, the running sum and
  // max; piece 16 folds them into the segment state.  Few values are live at once.
  float e[4], run_sum = 0.f, run_mx = -INFINITY;
  bf16x8 pc0, pc1;
  auto fast_piece = [&](const f32x16& s, float nm, int k) {
    const int j = 2 * (k >> 2);
    switch (k < 16 ? (k & 3) : 4) {
      case 0:
        e[0] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], c, nm));
        e[1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j + 1], c, nm));
        break;
      case 1:
        e[2] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 + j], c, nm));
        e[3] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[9 + j], c, nm));
        break;
      case 2:
        put_p(pc0, j, pack_bf16x2(e[0], e[1]));
        put_p(pc1, j, pack_bf16x2(e[2], e[3]));
        break;
      case 3: {
        // the denominator sums the same bf16 weights that P.V multiplies
        const float sm = sum_bf16x2(get_p(pc0, j)) + sum_bf16x2(get_p(pc1, j));
        const float mx = fmaxf(fmaxf(s[j], s[j + 1]), fmaxf(s[8 + j], s[9 + j]));
        run_sum = (j == 0) ? sm : run_sum + sm;
        run_mx = (j == 0) ? mx : fmaxf(run_mx, mx);
        break;
      }
      default:
        if (k == 16) {
          st.lsum += run_sum;
          st.s_max = fmaxf(st.s_max, run_mx);
        }
        break;
    }
  };
  // Masked path: causal edge tiles, and the first tile (which sets the reference).
  auto masked_softmax = [&](f32x16 s, int t, uint32_t live) {
    float mx = -INFINITY;
    // this lane half's tokens start at 8h: shift once, so that each bit test
    // below has a constant position (no per-lane masks held in registers)
    const uint32_t live_h = live >> (8 * h);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int tk = 8 * h + 16 * (k >> 3) + (k & 7);  // token within the tile
      const bool vis = (t * TILE + tk) < n_vis && ((live_h >> (16 * (k >> 3) + (k & 7))) & 1u);
      const float v = vis ? s[k] * c : -INFINITY;
      s[k] = v;
      mx = fmaxf(mx, v);
    }
    mx = max_halves(mx);
    if (st.m_ref == -INFINITY) st.m_ref = mx;  // first tile with a visible token sets the reference
    st.m_max = fmaxf(st.m_max, mx);
    const float mbase = (st.m_ref == -INFINITY) ? 0.f : st.m_ref;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const uint32_t a = pack_bf16x2(__builtin_amdgcn_exp2f(s[j] - mbase), __builtin_amdgcn_exp2f(s[j + 1] - mbase));
      const uint32_t b2 = pack_bf16x2(__builtin_amdgcn_exp2f(s[8 + j] - mbase),
                                      __builtin_amdgcn_exp2f(s[9 + j] - mbase));
      put_p(pc0, j, a);
      put_p(pc1, j, b2);
      st.lsum += sum_bf16x2(a) + sum_bf16x2(b2);  // the bf16 weights P.V multiplies
    }
    st.ref_ready = __builtin_amdgcn_ballot_w64(st.m_ref == -INFINITY) == 0;
  };

  // The loop runs one tile ahead in QK^T: iteration t computes QK^T of tile t+1
  // with tile t's softmax between its MFMAs, exchanges P of tile t, then does
  // P.V of tile t.  Tiles t0 .. t0+2 are in flight on entry.
  wait_tile(t0, 2);
  wait_lgkm0();
  block_barrier();  // tile t0 is in LDS
  f32x16 s_next{};
  if (ACTIVE && OWN) s_next = qk(buf_of(t0), no_fill, no_pre);
  const TileLoad no_load{nullptr, 0u, 0u};
  for (int t = t0; t < t1; ++t) {
    const f32x16 s = s_next;
    TileLoad tl = no_load;
    // live rows of tile t (sparse layout: the shares' published bits; the
    // dense layouts mask by position only)
    uint32_t live = ~0u;
    if constexpr (PS == 0) {
      const __attribute__((address_space(3))) uint32_t* vm =
          (const __attribute__((address_space(3))) uint32_t*)((__attribute__((address_space(3))) uint8_t*)smem +
                                                               VMASK_OFF + (t & (IDX_SLOTS - 1)) * 4);
      live = uniform(*vm);
    }
    const bool fast = c_pos && st.ref_ready && (t + 1) * TILE <= min_vis && live == ~0u;
    if (t + 1 < t1) {
      wait_tile(t + 1, 1);
      wait_lgkm0();
      block_barrier();  // tile t+1 is in LDS; every wave is done with tile t-1's buffer
      // Tile t+3 goes to the buffer of tile t-1.  Even waves issue their share
      // now, odd waves at the P exchange below: two bursts of loads queue in the
      // CU's address unit instead of one burst from all four waves.
      // (active waves run this once the first A fragments of QK^T(t+1) are on
      // their way, so the tile preparation and the DMA issue overlap their
      // latency)
      auto load_ahead = [&] {
        if constexpr (PS == 0) {
          // sparse: every wave now, its share of tile t+3 then the entries of t+5
          if (t + 3 < t1) {
            issue_sparse_share<FP8>(p, smem, buf_of(t + 3), t + 3);
            issue_sparse_index(p, smem, b, t + 5, t + 5 < t1);
          }
        } else {
          if (t + 3 < t1) {
            tl = prepare_tile<FP8, PS>(p, smem, buf_of(t + 3), b, L, t + 3, pw);
            if ((w & 1) == 0 || !ACTIVE) {
              issue_tile_share<FP8>(tl);
              tl = no_load;
            }
          }
        }
      };
      if (!ACTIVE || !OWN) load_ahead();
      if (ACTIVE && OWN) {
        if (fast && (!FP8 || Q8)) {
          const float nm = -st.m_ref;
          s_next = qk(buf_of(t + 1), [&](int k) { fast_piece(s, nm, k); }, load_ahead);
        } else if (fast) {
          // fp8: the A operands' widening already fills the VALU slots between
          // the MFMAs, so the softmax goes first
          const float nm = -st.m_ref;
#pragma unroll
          for (int k = 0; k < QK_STEPS; ++k) fast_piece(s, nm, k);
          s_next = qk(buf_of(t + 1), no_fill, load_ahead);
        } else {
          masked_softmax(s, t, live);
          s_next = qk(buf_of(t + 1), no_fill, load_ahead);
        }
      }
    } else if (ACTIVE && OWN) {
      if (fast) {
        const float nm = -st.m_ref;
#pragma unroll
        for (int k = 0; k < QK_STEPS; ++k) fast_piece(s, nm, k);
      } else {
        masked_softmax(s, t, live);
      }
    }
    if (!ACTIVE) {
      wait_lgkm0();
      block_barrier();  // P of tile t posted
      continue;
    }
    // ---------------- P exchange: the partner wave (w ^ 1) owns the other 32
    // pairs of this 64-pair group; each wave posts its P and reads the
    // partner's.  The P write goes first and the barrier waits for it alone:
    // the first V^T fragments, read after it, stay in flight across the
    // barrier (their latency overlaps the barrier and the odd waves' DMA).
    const uint32_t buf = opaque(buf_of(t));
    constexpr int GV = 4;  // V^T fragments read this many steps ahead
    constexpr int V_READS = GV * (FP8 ? 1 : 2);  // LDS reads of those fragments
    *(__attribute__((address_space(3))) bf16x8*)((__attribute__((address_space(3))) uint8_t*)smem + ps_own) = pc0;
    *(__attribute__((address_space(3))) bf16x8*)((__attribute__((address_space(3))) uint8_t*)smem + ps_own + 1024) =
        pc1;
    asm volatile("" ::: "memory");  // the P write stays ahead of the V^T reads
    u32x4 vraw[GV];
#pragma unroll
    for (int i = 0; i < GV; ++i) vraw[i] = load_v(buf, i);
    issue_tile_share<FP8>(tl);
    wait_lgkm<V_READS>();  // the two P writes have landed
    block_barrier();  // P of tile t posted
    const bf16x8 pp0 = *(const __attribute__((address_space(3))) bf16x8*)(
        (const __attribute__((address_space(3))) uint8_t*)smem + ps_other);
    const bf16x8 pp1 = *(const __attribute__((address_space(3))) bf16x8*)(
        (const __attribute__((address_space(3))) uint8_t*)smem + ps_other + 1024);
    // ---------------- O^T (this wave's 256 dims) += V^T . P^T for the wave's own
    // 32 pairs (acc[2d]) and the partner's (acc[2d + 1]): each V^T fragment
    // feeds two MFMAs.  The own-P MFMAs of the first GV steps go first, while
    // the partner's P is still on its way.  A half with no live pair is skipped.
    if constexpr (OWN) {
#pragma unroll
      for (int step = 0; step < GV; ++step)
        mfma_acc_agpr<FP8>(st.acc[2 * (step & 7)], to_bf16(vraw[step]), pc0);
    }
#pragma unroll
    for (int step = 0; step < PV_BLOCKS; ++step) {
      const int d = step & 7;
      const bf16x8 v = to_bf16(vraw[step % GV]);
      if constexpr (OWN) {
        if (step >= GV) mfma_acc_agpr<FP8>(st.acc[2 * d], v, (step >> 3) ? pc1 : pc0);
      }
      if constexpr (PARTNER) mfma_acc_agpr<FP8>(st.acc[2 * d + 1], v, (step >> 3) ? pp1 : pp0);
      if (step + GV < PV_BLOCKS) vraw[step % GV] = load_v(buf, step + GV);
    }
    // results land before anything but the next tile's MFMAs can touch them
    // (the compiler may copy the accumulators once the loop exits)
    asm volatile("s_nop 7\n\ts_nop 3" ::: "memory");
  }
}

// Returns false when the segment has to be redone: some logit beat its lane's
// reference max (the first visible tile's max) by more than 2^32.  m_seed then
// holds each lane's observed max as the new reference and the caller runs the
// segment again, which cannot overflow; O is never rescaled.
template <bool FP8, int PS, int QM>
__device__ __forceinline__ bool process_segment(const Params& p, uint8_t* smem, int b, int pb, int L, int t0, int t1,
                                                int slot, float& m_seed) {
  // (an opaque thread id: lane-derived values are recomputed for every
  // segment instead of being held, or spilled, across the whole kernel)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int h = lane >> 5;
  const int col = lane & 31;
  int r0;
  const int qb = request_rows(p, b, r0);
  const int H = p.heads;
  const int npairs = qb * H;
  const int pair0 = pb * PAIRS_BLOCK + w * PAIRS_WAVE;  // first pair of this wave's QK^T
  const int pair = pair0 + col;
  const bool valid = pair < npairs;
  // a 64-pair group (waves 2g, 2g+1) runs when any of its pairs is live: the
  // wave that holds its QK^T pairs and the partner that shares its P.V
  const int gpair0 = pb * PAIRS_BLOCK + (w >> 1) * 2 * PAIRS_WAVE;
  const bool active = gpair0 < npairs;  // wave-uniform, same for both waves of the group
  const int qi = valid ? pair / H : 0;
  const int head = valid ? pair - qi * H : 0;
  // visible rows: causal rows see L - q_b + qi + 1; inactive lanes see L (their
  // zero query gives finite logits and their results are discarded)
  const int n_vis = !valid ? L : visible_rows(p, b, L, qb, qi);
  // (rows see more as qi grows, so the wave's first pair sees the fewest)
  const int min_vis = uniform(pair0 < npairs ? visible_rows(p, b, L, qb, pair0 / H) : L);

  // page ids of the segment, then the first three tiles in flight before the
  // query loads
  PageWin pw{0, 0, 0};
  if constexpr (PS == 0) {
    // sparse: the list entries of the first four tiles (one ring slot each),
    // then (landed) the first three tiles' rows, then the entries of the
    // fifth, into the slot the first has just been read from
#pragma unroll
    for (int k = 0; k < IDX_SLOTS; ++k) issue_sparse_index(p, smem, b, t0 + k, t0 + k < t1);
    wait_vmcnt<0>();
    issue_sparse_share<FP8>(p, smem, 0, t0);
    if (t0 + 1 < t1) issue_sparse_share<FP8>(p, smem, TILEB, t0 + 1);
    if (t0 + 2 < t1) issue_sparse_share<FP8>(p, smem, 2 * TILEB, t0 + 2);
    issue_sparse_index(p, smem, b, t0 + 4, t0 + 4 < t1);
  } else {
    load_page_window<page_window<FP8>()>(p, b, ceil_div(L, PS), uniform((t0 * TILE) / PS), pw);
    issue_tile<FP8, PS>(p, smem, 0, b, L, t0, pw);
    if (t0 + 1 < t1) issue_tile<FP8, PS>(p, smem, TILEB, b, L, t0 + 1, pw);
    if (t0 + 2 < t1) issue_tile<FP8, PS>(p, smem, 2 * TILEB, b, L, t0 + 2, pw);
  }

  // Query fragments (B operand): lane holds pair `col`.  bf16: step kk < 32
  // covers latent dims 16kk + 8h .. +8, steps 32..35 RoPE dims 512 + 16(kk-32)
  // + 8h.  fp8 query: step kk < 9 covers bytes 64kk + 32h .. +32 of the row.
  constexpr bool Q8 = QM != 0;
  constexpr int QN = QM == 2 ? 18 : Q8 ? 9 : QK_STEPS;
  using QFrag = std::conditional_t<Q8, i32x8, bf16x8>;
  QFrag qf[QN];
  float c = p.scale_log2;
  {
    const bool live = valid && active;
    if constexpr (QM == 2) {
      // Split query: fragment k < 9 is dims 64k + 32h .. +32 of the row (the
      // fp8 query's layout), qf[k] holding q_hi and qf[9 + k] q_lo of
      // q 2^e = q_hi + q_lo, with 2^e putting the pair's largest |q| in
      // [128, 256).  A bf16 value has 8 significant bits: q_hi keeps the top
      // four, the remainder has at most four and is exact in E4M3 unless it
      // falls below E4M3's subnormal step 2^-9 (only for |q 2^e| < 2^-2, i.e.
      // elements under 2^-9 of the pair's largest), where the error is at most
      // 2^-10, i.e. 2^-17 of the pair's largest.  The scores come out times 2^e,
      // which the lane's c takes back out.  The row is read twice (max, then
      // split) so that the raw values never sit beside the fragments.
      const uint16_t* qrow = p.q + ((size_t)(r0 + qi) * H + head) * D_QK + 32 * h;
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < 9; ++k) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 v = live ? *(const u32x4*)(qrow + 64 * k + 8 * j) : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(__uint_as_float(v[i] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(v[i] & 0xffff0000u)));
          }
        }
      }
      amax = max_halves(amax);
      const int e = 8 - __builtin_amdgcn_frexp_expf(amax);
      c = __builtin_amdgcn_ldexpf(p.scale_log2, -e);
      // a positive scale stays positive in every lane (the fast-path test
      // must agree across the wave): at worst the smallest normal float, where
      // the logits are below 2^-100 and were smaller still
      if (p.scale_log2 > 0.f) c = fmaxf(c, 1.17549435e-38f);
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        i32x8 hi8, lo8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 v = live ? *(const u32x4*)(qrow + 64 * k + 8 * j) : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2) {
            // word 2j + i2 holds dims 8j + 4i2 .. +4: values v[2i2] (bytes 0-1)
            // and v[2i2 + 1] (bytes 2-3), each a pair of bf16
            const float a0 = __builtin_amdgcn_ldexpf(__uint_as_float(v[2 * i2] << 16), e);
            const float b0 = __builtin_amdgcn_ldexpf(__uint_as_float(v[2 * i2] & 0xffff0000u), e);
            const float a1 = __builtin_amdgcn_ldexpf(__uint_as_float(v[2 * i2 + 1] << 16), e);
            const float b1 = __builtin_amdgcn_ldexpf(__uint_as_float(v[2 * i2 + 1] & 0xffff0000u), e);
            int hw = __builtin_amdgcn_cvt_pk_fp8_f32(a0, b0, 0, false);
            hw = __builtin_amdgcn_cvt_pk_fp8_f32(a1, b1, hw, true);
            const f32x2 r0 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
            const f32x2 r1 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
            int lw = __builtin_amdgcn_cvt_pk_fp8_f32(a0 - r0[0], b0 - r0[1], 0, false);
            lw = __builtin_amdgcn_cvt_pk_fp8_f32(a1 - r1[0], b1 - r1[1], lw, true);
            hi8[2 * j + i2] = hw;
            lo8[2 * j + i2] = lw;
          }
        }
        qf[k] = hi8;
        qf[9 + k] = lo8;
      }
    } else if constexpr (Q8) {
      const uint8_t* qrow = (const uint8_t*)p.q + ((size_t)(r0 + qi) * H + head) * D_QK + 32 * h;
#pragma unroll
      for (int k = 0; k < QN; ++k) {
        const u32x4 x = live ? *(const u32x4*)(qrow + 64 * k) : u32x4{0, 0, 0, 0};
        const u32x4 y = live ? *(const u32x4*)(qrow + 64 * k + 16) : u32x4{0, 0, 0, 0};
        qf[k] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
      }
    } else {
      const uint16_t* qrow = p.q + ((size_t)(r0 + qi) * H + head) * D_QK + 8 * h;
#pragma unroll
      for (int k = 0; k < QN; ++k) {
        const u32x4 v = live ? *(const u32x4*)(qrow + 16 * k) : u32x4{0, 0, 0, 0};
        qf[k] = __builtin_bit_cast(bf16x8, v);
      }
    }
    // Wait for the loads here and redefine the registers through an empty asm,
    // so the compiler sees no load pending on them inside the tile loop (a
    // vmcnt wait there would also drain the tiles' DMA).
    drain_vector_loads();
#pragma unroll
    for (int k = 0; k < QN; ++k) asm volatile("" : "+v"(qf[k]));
  }

  SegState st;
#pragma unroll
  for (int i = 0; i < PV_BLOCKS; ++i) st.acc[i] = f32x16{};
  st.m_ref = m_seed;
  st.m_max = m_seed;
  st.s_max = -INFINITY;
  st.lsum = 0.f;
  st.ref_ready = __builtin_amdgcn_ballot_w64(m_seed == -INFINITY) == 0;
  const bool own_live = pair0 < npairs;
  const bool partner_live = pb * PAIRS_BLOCK + (w ^ 1) * PAIRS_WAVE < npairs;
  if (active && own_live && partner_live)
    segment_loop<FP8, PS, true, QM, true, true>(p, smem, b, L, t0, t1, qf, c, n_vis, min_vis, st, pw);
  else if (active && own_live)
    segment_loop<FP8, PS, true, QM, true, false>(p, smem, b, L, t0, t1, qf, c, n_vis, min_vis, st, pw);
  else if (active)
    segment_loop<FP8, PS, true, QM, false, true>(p, smem, b, L, t0, t1, qf, c, n_vis, min_vis, st, pw);
  else segment_loop<FP8, PS, false, QM, false, false>(p, smem, b, L, t0, t1, qf, c, n_vis, min_vis, st, pw);

  // ---- segment end: the largest logit of the segment decides whether some
  // exponential went past the threshold; all waves idle on LDS; one flag per
  // wave says "redo"
  const float fast_max = (st.s_max == -INFINITY) ? -INFINITY : max_halves(st.s_max) * c;
  const float m_max = fmaxf(st.m_max, fast_max);
  const bool over = m_max > st.m_ref + RESCALE_THRESHOLD;
  int* flags = (int*)(smem + FLAGS_OFF);
  wait_lgkm0();
  block_barrier();
  if (lane == 0) flags[w] = __builtin_amdgcn_ballot_w64(over) != 0 ? 1 : 0;
  wait_lgkm0();
  block_barrier();
  if (uniform(flags[0] | flags[1] | flags[2] | flags[3]) != 0) {
    m_seed = m_max;
    return false;
  }

  // ---------------- epilogue.  O goes out unnormalised as bf16 (its scale is
  // relative to m_ref; the merge kernel divides by the summed denominator).
  // It is staged in LDS (the tile buffers are all consumed) as the unit's
  // [128 pairs][512 dims] block, 16-byte chunk c of row r at chunk c ^ (r & 15),
  // so that each wave then stores whole 1 KB rows.  Each accumulator is read
  // out of its AGPR once and pairs of values go to bf16 in one conversion.
  const float lsum = sum_halves(st.lsum);
  if (active) {
    const int dh = w & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // acc[2d] holds this wave's own 32 pairs, acc[2d + 1] its partner's
      const int r = (w >> 1) * 2 * PAIRS_WAVE + (j ^ (w & 1)) * PAIRS_WAVE + col;  // pair within the unit
      const uint32_t rowb = (uint32_t)r * (D_V * 2) + 8 * h;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const f32x16 v = st.acc[2 * d + j];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          // lane holds dims 256 dh + 32 d + 8 q4 + 4 h .. +4: chunk 32 dh + 4 d + q4
          const int chunk = 32 * dh + 4 * d + q4;
          u32x2 packed;
#pragma unroll
          for (int e = 0; e < 2; ++e) packed[e] = pack_bf16x2(v[4 * q4 + 2 * e], v[4 * q4 + 2 * e + 1]);
          *(__attribute__((address_space(3))) u32x2*)((__attribute__((address_space(3))) uint8_t*)smem + rowb +
                                                     16 * (chunk ^ (r & 15))) = packed;
        }
      }
    }
  }
  if (h == 0 && valid) {
    float* ml = p.ws_ml + ((size_t)slot * PAIRS_BLOCK + w * PAIRS_WAVE + col) * 2;
    ml[0] = st.m_ref;
    ml[1] = lsum;
  }
  wait_lgkm0();
  block_barrier();  // the O block is in LDS
  // wave w stores rows [32 w, 32 w + 32), eight at a time, 16 bytes per lane
  uint16_t* wo = p.ws_o + (size_t)slot * PAIRS_BLOCK * D_V + 8 * lane;
#pragma unroll
  for (int r8 = 0; r8 < PAIRS_WAVE; r8 += 8) {
    u32x4 rows[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = w * PAIRS_WAVE + r8 + i;
      rows[i] = lds_read_b128(smem, (uint32_t)r * (D_V * 2) + 16 * (lane ^ (r & 15)));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = w * PAIRS_WAVE + r8 + i;
      if (pb * PAIRS_BLOCK + r < npairs) *(u32x4*)(wo + (size_t)r * D_V) = rows[i];
    }
  }
  wait_lgkm0();
  block_barrier();  // LDS is free for the next segment's tiles
  return true;
}

// ---------------------------------------------------------------- decode kernel

template <bool FP8, int PS, int QM>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_kernel(Params p) {
  if (p.bmm1_dev != nullptr) p.scale_log2 = *p.bmm1_dev * LOG2E;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  // The plan lives in LDS only until this workgroup has found its starting point.
  int* tile_off = (int*)(smem + PLAN_SCRATCH_OFF);
  int* unit_off = (int*)(smem + UNIT_SCRATCH_OFF);
  const int GU = uniform(build_plan(p, tile_off, unit_off, (int*)(smem + SCAN_SCRATCH_OFF)));
  const int B = p.batch;
  const int S0 = p.seg_cost;
  // Cost space: unit u (request b, pair block pb) takes S0 + T_b consecutive
  // positions, S0 for the segment start it forces and then one per tile, so
  // tile t of u sits at tile_off[b] + pb T_b + t + (u + 1) S0.  Cost range k
  // takes the positions [k C, (k + 1) C): equal cost, counting each extra
  // segment.  Normally each workgroup walks a range of its own.  With groups
  // (GU > 1: every request holds the same GU pair blocks) a cost unit is a
  // whole request, and the GU workgroups of a group, on one XCD, walk the same
  // range together, workgroup j doing pair block j of each request: they read
  // each KV tile at about the same time, so all but the first read hit L2.
  const int TC = uniform(tile_off[B] + unit_off[B] * S0);
  const int G = p.grid;
  const int C = max(1, ceil_div(TC, G / GU));
  if (blockIdx.x == 0) {
    for (int b = threadIdx.x; b <= B; b += THREADS) {
      p.ws_plan[2 + b] = tile_off[b];
      p.ws_plan[3 + B + b] = unit_off[b];
    }
    if (threadIdx.x == 0) {
      p.ws_plan[0] = C;
      p.ws_plan[1] = GU;
    }
  }
  // Consecutive logical workgroups sit on one XCD (dispatch is round-robin over
  // the 8 XCDs), so workgroups sharing a request's KV share an L2.
  const int i = blockIdx.x;
  const int gw = (G % 8 == 0) ? ((i & 7) * (G >> 3) + (i >> 3)) : i;
  const int g = gw / GU;        // this workgroup's cost range
  const int q = gw - g * GU;    // its pair block of every request in the range (groups)
  int x = g * C;
  const int end = min(TC, x + C);
  int b = 0, rel = 0;
  if (x < end) {
    int lo = 0, hi = B;  // cost offset of request lo <= x < that of request hi
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_off[mid] + unit_off[mid] * S0 <= x) lo = mid; else hi = mid;
    }
    b = lo;
    rel = x - (tile_off[lo] + unit_off[lo] * S0);
  }
  b = uniform(b);
  rel = uniform(rel);
  int u_base = uniform(unit_off[b]);  // global unit index of request b's first unit
  __syncthreads();  // the LDS plan is dead from here on
  while (x < end) {
    // walk the cost space forward from request b
    const int L = uniform(req_len(p, b));
    int r0;
    const int qb = uniform(request_rows(p, b, r0));
    const int T = uniform(request_tiles(p, b));
    const int units = uniform(GU > 1 ? min(request_units(p, qb), 1) : request_units(p, qb));  // cost units
    const int span = S0 + T;
    if (T == 0 || units == 0) {  // nothing to compute (lengths outside the contract)
      x += units * S0 - rel;
      rel = 0;
      ++b;
      u_base += units;
      continue;
    }
    const int pb = rel / span;
    int r = rel - pb * span;
    if (r < S0) {  // a unit's start: its tiles begin S0 - r positions on
      x += S0 - r;
      rel += S0 - r;
      r = S0;
      if (x >= end) break;
    }
    const int t0 = r - S0;
    const int t1 = min(T, t0 + (end - x));
    // segment (cost range g, cost unit u) has slot (g + u) GU + q: unique, since
    // every later segment of a range has a larger g or a larger u, and the
    // workgroups of a group differ in q
    const int slot = (g + u_base + pb) * GU + q;
    float m_seed = -INFINITY;
    while (!process_segment<FP8, PS, QM>(p, smem, b, GU > 1 ? q : pb, L, t0, t1, slot, m_seed)) {
    }
    x += t1 - t0;
    rel += t1 - t0;
    if (rel >= units * span) {
      ++b;
      rel = 0;
      u_base += units;
    }
  }
}

// ---------------------------------------------------------------- split merge

// Max / sum over the 64 lanes of a wave, result in every lane.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One wave per (query row, head): combine the segments of its unit,
// M = max_s m_s, w_s = 2^(m_s - M), out = bmm2 * sum w_s O_s / sum w_s l_s,
// lse = ln2 * (M + log2 sum w_s l_s).  A unit done by one workgroup has a single
// segment (w = 1): the same formula normalises it.  The loads of all segments'
// (max, sum) and of eight segments' O are in flight together: the kernel is
// bound by memory latency otherwise.  The summation order is fixed.
__global__ __launch_bounds__(MERGE_THREADS) void mla_merge_kernel(Params p) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * (MERGE_THREADS / 64) + (threadIdx.x >> 6);
  const int H = p.heads;
  if (item >= p.total_q * H) return;
  const int row = item / H;
  const int head = item - row * H;
  int b;
  if (p.qo_indptr != nullptr) {
    // the row's request, lane-parallel in one round trip: qo_indptr starts at
    // 0 and increases strictly, so b + 1 entries of [0, B) are <= row
    int cnt = 0;
    for (int c0 = 0; c0 < p.batch; c0 += 128) {
      const int j0 = c0 + lane, j1 = c0 + 64 + lane;
      const bool in0 = j0 < p.batch && p.qo_indptr[j0] <= row;
      const bool in1 = j1 < p.batch && p.qo_indptr[j1] <= row;
      cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(in0)) +
             __builtin_popcountll(__builtin_amdgcn_ballot_w64(in1));
    }
    b = uniform(cnt - 1);
  } else {
    b = row / p.q_len_fixed;
  }
  // everything the segment addresses depend on, in one round trip
  const int r0 = p.qo_indptr != nullptr ? p.qo_indptr[b] : b * p.q_len_fixed;
  const int C = p.ws_plan[0];
  const int L = req_len(p, b);
  const int tile_off = p.ws_plan[2 + b];
  const int unit_off = p.ws_plan[3 + p.batch + b];
  const int pair = (row - r0) * H + head;
  const int pb = pair / PAIRS_BLOCK;
  const int pl = pair - pb * PAIRS_BLOCK;
  const int T = max(0, ceil_div(L, TILE));
  // with workgroup groups the request is one cost unit and pb picks the
  // group member (slot offset q); otherwise pb is part of the cost position
  const int GU = p.ws_plan[1];
  const int pbc = GU > 1 ? 0 : pb;
  const int q = pb - pbc;
  const int u = unit_off + pbc;
  const int U0 = tile_off + pbc * T + (u + 1) * p.seg_cost;  // cost position of the unit's first tile
  const int g0 = U0 / C;
  const int g1 = (U0 + T - 1) / C;
  const int nseg = (T > 0) ? g1 - g0 + 1 : 0;  // a request with no rows (a sequence shard may have none) has no segment
  // segment s of the unit (cost range g0 + s) has slot (g0 + s + u) GU + q
  const size_t slot0 = (size_t)(g0 + u) * GU + q;
  const float* mlb = p.ws_ml + (slot0 * PAIRS_BLOCK + pl) * 2;
  const uint16_t* ob = p.ws_o + (slot0 * PAIRS_BLOCK + pl) * D_V + 8 * lane;
  // One round trip before any arithmetic: the O rows of the first MB segments
  // and the (max, sum) of the first 64 (one per lane) are all in flight
  // together; lane l holds dims 8l .. 8l + 8 of each O row.
  constexpr int MB = 7;  // O rows in flight (61 VGPRs: 8 waves per SIMD, all a SIMD holds)
  // a sink is one more softmax term with no value row: it joins the max and
  // the denominator
  const float sink = (p.sinks != nullptr) ? p.sinks[head] * LOG2E : -INFINITY;
  const size_t o_step = (size_t)GU * PAIRS_BLOCK * D_V;
  const size_t ml_step = (size_t)GU * PAIRS_BLOCK * 2;
  u32x4 o[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
    if (i < nseg) o[i] = *(const u32x4*)(ob + (size_t)i * o_step);
  float m_first = -INFINITY, s_first = 0.f;
  if (lane < nseg) {
    m_first = mlb[(size_t)lane * ml_step];
    s_first = mlb[(size_t)lane * ml_step + 1];
  }
  float M = m_first;
  for (int c0 = 64; c0 < nseg; c0 += 64) {
    if (c0 + lane < nseg) M = fmaxf(M, mlb[(size_t)(c0 + lane) * ml_step]);
  }
  M = wave_max(M);
  M = fmaxf(M, sink);
  float den = 0.f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int c0 = 0; c0 < nseg; c0 += 64) {
    float wl = 0.f;  // this lane's segment weight 2^(m - M)
    if (c0 + lane < nseg) {
      float m = m_first, sv = s_first;
      if (c0 > 0) {
        m = mlb[(size_t)(c0 + lane) * ml_step];
        sv = mlb[(size_t)(c0 + lane) * ml_step + 1];
      }
      wl = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M);
      den += wl * sv;
    }
    const int cn = min(64, nseg - c0);
    for (int s0 = 0; s0 < cn; s0 += MB) {
      if (c0 + s0 > 0) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
          if (s0 + i < cn) o[i] = *(const u32x4*)(ob + (size_t)(c0 + s0 + i) * o_step);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if (s0 + i < cn) {
          const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s0 + i));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += w * __uint_as_float(o[i][e] << 16);
            acc[2 * e + 1] += w * __uint_as_float(o[i][e] & 0xffff0000u);
          }
        }
      }
    }
  }
  den = wave_sum(den);
  if (sink != -INFINITY) den += __builtin_amdgcn_exp2f(sink - M);
  // a (row, head) that sees no row (possible only for a sequence shard) gets
  // out = 0 and lse = -inf
  const bool empty = !(den > 0.f);
  const float inv = empty ? 0.f : ((p.bmm2_dev != nullptr) ? *p.bmm2_dev : p.bmm2) / den;
  u32x4 packed;
#pragma unroll
  for (int e = 0; e < 4; ++e) packed[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *(u32x4*)(p.out + (size_t)item * D_V + 8 * lane) = packed;
  if (p.lse != nullptr && lane == 0) p.lse[item] = empty ? -INFINITY : (M + __log2f(den)) * LN2;
}

// Combine G partial results of the same items (the shards of a sequence-
// sharded decode): M = max_g lse_g, w_g = exp(lse_g - M), out = sum w_g out_g /
// sum w_g, lse = M + ln sum w_g.  One wave per item, lane l holding dims
// 8l .. 8l + 8; the lse of up to 64 partials load at once, one per lane.
__global__ __launch_bounds__(MERGE_THREADS) void mla_merge_partials_kernel(const uint16_t* outs, const float* lses,
                                                                           int G, int64_t items, uint16_t* out,
                                                                           float* lse) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * (MERGE_THREADS / 64) + (threadIdx.x >> 6);
  if (item >= items) return;
  float M = -INFINITY;
  for (int c0 = 0; c0 < G; c0 += 64)
    if (c0 + lane < G) M = fmaxf(M, lses[(int64_t)(c0 + lane) * items + item]);
  M = wave_max(M);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float den = 0.f;
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < G; c0 += 64) {
      float wl = 0.f;
      if (c0 + lane < G) {
        const float l = lses[(int64_t)(c0 + lane) * items + item];
        wl = (l == -INFINITY) ? 0.f : __expf(l - M);
        den += wl;
      }
      const int cn = min(64, G - c0);
      for (int g = 0; g < cn; ++g) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), g));
        if (w == 0.f) continue;  // wave-uniform: an empty partial adds nothing
        const u32x4 o = *(const u32x4*)(outs + ((int64_t)(c0 + g) * items + item) * D_V + 8 * lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += w * __uint_as_float(o[e] << 16);
          acc[2 * e + 1] += w * __uint_as_float(o[e] & 0xffff0000u);
        }
      }
    }
    den = wave_sum(den);
  }
  const bool empty = !(den > 0.f);
  const float inv = empty ? 0.f : 1.f / den;
  u32x4 packed;
#pragma unroll
  for (int e = 0; e < 4; ++e) packed[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *(u32x4*)(out + item * D_V + 8 * lane) = packed;
  if (lse != nullptr && lane == 0) lse[item] = empty ? -INFINITY : M + __logf(den);
}

// Contract check (FlashInfer docs, "prims_ts_batch_decode_with_kv_cache_mla",
// contract paragraph: the part of a launch's contract held in device memory).
// One workgroup: every thread takes requests b = tid, tid + 1024, ... for the
// length and offset rules, then the block-table entries a launch would read
// (0 .. ceil(L_b / page_size) - 1, at most the row's width), 1024 at a time.
// Violation bits and the lowest offending request meet in LDS; thread 0
// writes result[0] = bits, result[1] = that request + 1 (0: none).
struct ContractArgs {
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qo_indptr;
  uint32_t* result;
  int64_t num_pages;
  int32_t batch, bt_stride, page_size, max_seq_len, max_q_len, q_len_fixed, total_q, causal;
};

constexpr int CHECK_THREADS = 1024;

__global__ __launch_bounds__(CHECK_THREADS) void mla_check_contract_kernel(ContractArgs c) {
  __shared__ uint32_t s_bits;
  __shared__ int s_first;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_bits = 0;
    s_first = c.batch;
  }
  __syncthreads();
  uint32_t bits = 0;
  int first = c.batch;
  for (int b = tid; b < c.batch; b += CHECK_THREADS) {
    uint32_t v = 0;
    const int L = c.seq_lens[b];
    if (L < 1 || L > c.max_seq_len) v |= MLA_CONTRACT_SEQ_LEN;
    int qb = c.q_len_fixed;
    if (c.qo_indptr != nullptr) {
      const int a = c.qo_indptr[b], e = c.qo_indptr[b + 1];
      if (b == 0 && a != 0) v |= MLA_CONTRACT_QO_START;
      if (e <= a) v |= MLA_CONTRACT_QO_ORDER;
      if (b == c.batch - 1 && e != c.total_q) v |= MLA_CONTRACT_QO_END;
      qb = e - a;
    }
    if (qb > c.max_q_len) v |= MLA_CONTRACT_Q_LEN;
    if (c.causal && qb > L) v |= MLA_CONTRACT_CAUSAL;
    if (v != 0) {
      bits |= v;
      first = min(first, b);
    }
  }
  for (int b = 0; b < c.batch; ++b) {
    const int64_t L = max(c.seq_lens[b], 0);
    const int np = (int)min((L + c.page_size - 1) / c.page_size, (int64_t)c.bt_stride);
    const int32_t* row = c.block_tables + (size_t)b * c.bt_stride;
    for (int j = tid; j < np; j += CHECK_THREADS) {
      const int32_t id = row[j];
      if (id < 0 || (int64_t)id >= c.num_pages) {
        bits |= MLA_CONTRACT_PAGE_ID;
        first = min(first, b);
      }
    }
  }
  if (bits != 0) {
    atomicOr(&s_bits, bits);
    atomicMin(&s_first, first);
  }
  __syncthreads();
  if (tid == 0) {
    c.result[0] = s_bits;
    c.result[1] = s_first < c.batch ? (uint32_t)s_first + 1u : 0u;
  }
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
std::atomic<int> g_seg_cost{-1};  // negative: the layout's default
std::atomic<int> g_groups{1};     // 0: never walk a cost range with a group of workgroups
std::atomic<void*> g_ev_start{nullptr};
std::atomic<void*> g_ev_decode{nullptr};
std::atomic<void*> g_ev_stop{nullptr};

// The workspace of mla_decode_paged_noalloc, one copy per device.  Host code
// never passes the array's name to a kernel: it looks up each device's
// address once (noalloc_scratch) and passes that.
__device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[MAX_DEVICES];
std::mutex g_scratch_mutex;

// Device address of this device's scratch array (looked up on its first use,
// with the device current), or null on failure.
void* noalloc_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
    p = addr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

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

// Upper bound on the units of a launch: every request has at most max_q_len rows.
int64_t max_units(const mla_decode_dims_t* d, int32_t max_q_len) {
  return (int64_t)d->batch * (((int64_t)max_q_len * d->num_heads + PAIRS_BLOCK - 1) / PAIRS_BLOCK);
}

WsLayout workspace_layout(int grid, int64_t units) {
  WsLayout l;
  auto align = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t slots = (size_t)grid + (size_t)units;
  l.plan_off = 0;
  l.ml_off = align((size_t)(3 + 2 * PLAN_INTS) * 4);
  l.o_off = align(l.ml_off + slots * PAIRS_BLOCK * 2 * 4);
  l.total = align(l.o_off + slots * PAIRS_BLOCK * D_V * 2);
  return l;
}

// Checks shared by the paged and the sparse layouts.
int validate_common(const mla_decode_dims_t* d) {
  if (d->num_heads <= 0 || d->num_heads % 16 != 0) return MLA_ERR_BAD_HEADS;
  // (row, head) items are counted in 32 bits by the merge launch
  if ((int64_t)d->total_q * d->num_heads >= ((int64_t)1 << 31) - 4) return MLA_ERR_BAD_SHAPE;
  if (d->page_size != 16 && d->page_size != 32 && d->page_size != 64) return MLA_ERR_BAD_PAGE_SIZE;
  if (d->kv_lora_rank != 512 || d->qk_rope_head_dim != 64) return MLA_ERR_BAD_HEAD_DIMS;
  if (d->kv_dtype != MLA_KV_BF16 && d->kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_BAD_DTYPE;
  return MLA_OK;
}

int validate(const mla_decode_dims_t* d, int32_t max_seq_len, int32_t max_q_len, bool packed) {
  if (d == nullptr) return MLA_ERR_NULL_POINTER;
  if (d->batch < 1 || d->batch > MLA_MAX_BATCH || max_seq_len < 1 || d->num_pages < 1) return MLA_ERR_BAD_SHAPE;
  const int c = validate_common(d);
  if (c != MLA_OK) return c;
  if (max_q_len < 1 || d->total_q < 1) return MLA_ERR_BAD_Q_LEN;
  if (!packed && (d->q_len_fixed != max_q_len || (int64_t)d->batch * d->q_len_fixed != d->total_q))
    return MLA_ERR_BAD_Q_LEN;
  if (packed && d->total_q > (int64_t)d->batch * max_q_len) return MLA_ERR_BAD_Q_LEN;
  if ((int64_t)d->block_table_stride * d->page_size < max_seq_len) return MLA_ERR_BAD_BLOCK_TABLE;
  // 32-bit cost arithmetic on device
  if (max_units(d, max_q_len) * ((max_seq_len + TILE - 1) / TILE + SEG_COST_MAX) >= (int64_t)1 << 30)
    return MLA_ERR_BAD_SHAPE;
  return MLA_OK;
}

// Sparse top-k layout: every query row is a unit group of its own.
int64_t sparse_units(const mla_decode_dims_t* d) {
  return (int64_t)d->total_q * ((d->num_heads + PAIRS_BLOCK - 1) / PAIRS_BLOCK);
}

int validate_sparse(const mla_decode_dims_t* d, int32_t top_k) {
  if (d == nullptr) return MLA_ERR_NULL_POINTER;
  const int c = validate_common(d);
  if (c != MLA_OK) return c;
  if (d->total_q < 1 || d->total_q > MLA_MAX_BATCH || d->num_pages < 1 || top_k < 1 || top_k > MLA_MAX_TOP_K)
    return MLA_ERR_BAD_SHAPE;
  if (d->block_table_stride < top_k) return MLA_ERR_BAD_BLOCK_TABLE;
  if (sparse_units(d) * ((top_k + TILE - 1) / TILE + SEG_COST_MAX) >= (int64_t)1 << 30) return MLA_ERR_BAD_SHAPE;
  return MLA_OK;
}

template <bool FP8, int PS, int QM>
void launch_decode(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL((mla_decode_kernel<FP8, PS, QM>), dim3(p.grid), dim3(THREADS), 0, s, p);
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
    case MLA_ERR_MISALIGNED: return "misaligned pointer (q, kv_cache, out, workspace: 16 bytes; lse, options: 4)";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than mla_decode_paged_workspace_size()";
    case MLA_ERR_BAD_Q_LEN: return "inconsistent query lengths (max_q_len, q_len_fixed, total_q)";
    case MLA_ERR_BAD_BLOCK_TABLE: return "block_table_stride * page_size < max_seq_len";
    case MLA_ERR_BAD_SHAPE: return "batch, max_seq_len or num_pages out of range";
    case MLA_ERR_HIP: return "HIP launch error";
    case MLA_ERR_NO_DEVICE: return "no usable HIP device";
    case MLA_ERR_SCRATCH_TOO_SMALL:
      return "mla_decode_paged_noalloc: the launch needs more workspace than MLA_NOALLOC_SCRATCH_BYTES";
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
  return workspace_layout(grid, max_units(dims, max_q_len)).total;
}

size_t mla_decode_paged_ex_workspace_size(const mla_decode_dims_t* dims, int32_t max_seq_len, int32_t max_q_len,
                                          int want_lse, const mla_decode_options_t* opts) {
  const int32_t top_k = opts != nullptr ? opts->sparse_top_k : 0;
  if (top_k <= 0) return mla_decode_paged_workspace_size(dims, max_seq_len, max_q_len, want_lse);
  if (dims == nullptr || validate_sparse(dims, top_k) != MLA_OK) return 0;
  int grid = 0;
  if (device_grid(&grid) != MLA_OK) return 0;
  return workspace_layout(grid, sparse_units(dims)).total;
}

int mla_decode_paged(const void* q, const void* kv_cache, const int32_t* block_tables, const int32_t* seq_lens,
                     const int32_t* qo_indptr, int32_t max_seq_len, int32_t max_q_len, float bmm1_scale,
                     float bmm2_scale, int causal, void* out, float* lse, void* workspace, size_t workspace_bytes,
                     const mla_decode_dims_t* dims, void* stream) {
  return mla_decode_paged_ex(q, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len, max_q_len, bmm1_scale,
                             bmm2_scale, causal, out, lse, workspace, workspace_bytes, dims, stream, nullptr);
}

int mla_decode_paged_ex(const void* q, const void* kv_cache, const int32_t* block_tables, const int32_t* seq_lens,
                        const int32_t* qo_indptr, int32_t max_seq_len, int32_t max_q_len, float bmm1_scale,
                        float bmm2_scale, int causal, void* out, float* lse, void* workspace, size_t workspace_bytes,
                        const mla_decode_dims_t* dims, void* stream, const mla_decode_options_t* opts) {
  const int32_t top_k = opts != nullptr ? opts->sparse_top_k : 0;
  const bool sparse = top_k > 0;
  const bool q8 = opts != nullptr && opts->q_fp8 != 0;
  if (!q || !kv_cache || !block_tables || (!seq_lens && !sparse) || !out || !workspace || !dims)
    return MLA_ERR_NULL_POINTER;
  if (opts != nullptr && (((uintptr_t)opts->bmm1_scale | (uintptr_t)opts->bmm2_scale | (uintptr_t)opts->sinks |
                            (uintptr_t)opts->seq_lens_global) & 3))
    return MLA_ERR_MISALIGNED;
  const bool dcp = opts != nullptr && opts->seq_lens_global != nullptr;
  if (dcp && (opts->cp_world < 1 || opts->cp_rank < 0 || opts->cp_rank >= opts->cp_world)) return MLA_ERR_BAD_SHAPE;
  if (dcp && lse == nullptr) return MLA_ERR_NULL_POINTER;
  if (top_k < 0 || (sparse && dcp) || (sparse && q8)) return MLA_ERR_BAD_SHAPE;
  const int v = sparse ? validate_sparse(dims, top_k) : validate(dims, max_seq_len, max_q_len, qo_indptr != nullptr);
  if (v != MLA_OK) return v;
  if (q8 && dims->kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_BAD_DTYPE;
  if (((uintptr_t)q | (uintptr_t)kv_cache | (uintptr_t)out | (uintptr_t)workspace) & 15) return MLA_ERR_MISALIGNED;
  if (lse != nullptr && ((uintptr_t)lse & 3)) return MLA_ERR_MISALIGNED;
  int grid = 0;
  const int gs = device_grid(&grid);
  if (gs != MLA_OK) return gs;
  const WsLayout wl = workspace_layout(grid, sparse ? sparse_units(dims) : max_units(dims, max_q_len));
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
  p.ws_o = (uint16_t*)(ws + wl.o_off);
  p.batch = dims->batch;
  p.heads = dims->num_heads;
  p.q_len_fixed = qo_indptr ? max_q_len : dims->q_len_fixed;
  p.total_q = dims->total_q;
  p.bt_stride = dims->block_table_stride;
  p.grid = grid;
  p.scale_log2 = bmm1_scale * LOG2E;
  p.bmm2 = bmm2_scale;
  p.causal = causal ? 1 : 0;
  const int seg_cost = g_seg_cost.load(std::memory_order_relaxed);
  p.seg_cost = seg_cost >= 0 ? seg_cost : (sparse ? SEG_COST_SPARSE : SEG_COST_DEFAULT);
  // The plan groups workgroups on the device when every request holds the
  // same U = 2, 4 or 8 pair blocks (see the work plan in the kernel).
  p.groups = (!sparse && g_groups.load(std::memory_order_relaxed) != 0) ? 1 : 0;
  p.bmm1_dev = opts ? opts->bmm1_scale : nullptr;
  p.bmm2_dev = opts ? opts->bmm2_scale : nullptr;
  // a sink is one softmax term per (row, head): in a sequence-sharded decode
  // rank 0's partial carries it, so merging the ranks counts it once
  p.sinks = (opts != nullptr && !(dcp && opts->cp_rank != 0)) ? opts->sinks : nullptr;
  p.seq_lens_global = dcp ? opts->seq_lens_global : nullptr;
  p.cp_world = dcp ? opts->cp_world : 1;
  p.cp_rank = dcp ? opts->cp_rank : 0;
  p.sparse_k = 0;
  if (sparse) {
    // each query row is a request of its own whose rows are its list entries
    p.batch = dims->total_q;
    p.q_len_fixed = 1;
    p.qo_indptr = nullptr;
    p.seq_lens = nullptr;
    p.causal = 0;
    p.sparse_k = top_k;
  }

  hipStream_t s = (hipStream_t)stream;
  const bool fp8 = dims->kv_dtype == MLA_KV_FP8_E4M3FN;
  void* ev0 = g_ev_start.load(std::memory_order_relaxed);
  void* evd = g_ev_decode.load(std::memory_order_relaxed);
  void* ev1 = g_ev_stop.load(std::memory_order_relaxed);
  if (ev0 != nullptr && ev1 != nullptr) (void)hipEventRecord((hipEvent_t)ev0, s);
  // fp8 cache: an fp8 query runs as given (mode 1), a bf16 query as two fp8
  // terms (mode 2); the sparse gather keeps the widened bf16 path (mode 0)
  if (sparse) {
    fp8 ? launch_decode<true, 0, 0>(p, s) : launch_decode<false, 0, 0>(p, s);
  } else if (fp8) {
    const int qm = q8 ? 1 : 2;
    switch (dims->page_size) {
      case 16: qm == 1 ? launch_decode<true, 16, 1>(p, s) : launch_decode<true, 16, 2>(p, s); break;
      case 32: qm == 1 ? launch_decode<true, 32, 1>(p, s) : launch_decode<true, 32, 2>(p, s); break;
      default: qm == 1 ? launch_decode<true, 64, 1>(p, s) : launch_decode<true, 64, 2>(p, s); break;
    }
  } else switch (dims->page_size) {
    case 16: launch_decode<false, 16, 0>(p, s); break;
    case 32: launch_decode<false, 32, 0>(p, s); break;
    default: launch_decode<false, 64, 0>(p, s); break;
  }
  if (ev0 != nullptr && ev1 != nullptr && evd != nullptr) (void)hipEventRecord((hipEvent_t)evd, s);
  const int items = dims->total_q * dims->num_heads;
  hipLaunchKernelGGL(mla_merge_kernel, dim3((items + 3) / 4), dim3(MERGE_THREADS), 0, s, p);
  if (ev0 != nullptr && ev1 != nullptr) (void)hipEventRecord((hipEvent_t)ev1, s);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_decode_paged_noalloc(const void* q, const void* kv_cache, const int32_t* block_tables,
                             const int32_t* seq_lens, const int32_t* qo_indptr, int32_t max_seq_len,
                             int32_t max_q_len, float bmm1_scale, float bmm2_scale, int causal, void* out,
                             float* lse, const mla_decode_dims_t* dims, void* stream) {
  if (dims == nullptr) return MLA_ERR_NULL_POINTER;
  const int v = validate(dims, max_seq_len, max_q_len, qo_indptr != nullptr);
  if (v != MLA_OK) return v;
  int grid = 0;
  const int gs = device_grid(&grid);
  if (gs != MLA_OK) return gs;
  const size_t need = workspace_layout(grid, max_units(dims, max_q_len)).total;
  if (need > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_SCRATCH_TOO_SMALL;
  void* ws = noalloc_scratch();
  if (ws == nullptr) return MLA_ERR_NO_DEVICE;
  return mla_decode_paged_ex(q, kv_cache, block_tables, seq_lens, qo_indptr, max_seq_len, max_q_len, bmm1_scale,
                             bmm2_scale, causal, out, lse, ws, MLA_NOALLOC_SCRATCH_BYTES, dims, stream, nullptr);
}

int mla_merge_partials(const void* outs, const float* lses, int32_t num_partials, int64_t items, void* out,
                       float* lse, void* stream) {
  if (!outs || !lses || !out) return MLA_ERR_NULL_POINTER;
  if (num_partials < 1 || items < 1) return MLA_ERR_BAD_SHAPE;
  if ((((uintptr_t)outs | (uintptr_t)out) & 15) || (((uintptr_t)lses | (uintptr_t)lse) & 3)) return MLA_ERR_MISALIGNED;
  const int64_t blocks = (items + MERGE_THREADS / 64 - 1) / (MERGE_THREADS / 64);
  if (blocks > 0x7fffffff) return MLA_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(mla_merge_partials_kernel, dim3((unsigned)blocks), dim3(MERGE_THREADS), 0, (hipStream_t)stream,
                     (const uint16_t*)outs, lses, (int)num_partials, items, (uint16_t*)out, lse);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_decode_check_contract(const int32_t* block_tables, const int32_t* seq_lens, const int32_t* qo_indptr,
                              int32_t max_seq_len, int32_t max_q_len, int causal, const mla_decode_dims_t* dims,
                              uint32_t* result, void* stream) {
  if (!block_tables || !seq_lens || !dims || !result) return MLA_ERR_NULL_POINTER;
  if ((uintptr_t)result & 3) return MLA_ERR_MISALIGNED;
  if (dims->batch < 1 || dims->batch > MLA_MAX_BATCH || dims->num_pages < 1 || dims->block_table_stride < 1 ||
      max_seq_len < 1)
    return MLA_ERR_BAD_SHAPE;
  if (dims->page_size != 16 && dims->page_size != 32 && dims->page_size != 64) return MLA_ERR_BAD_PAGE_SIZE;
  if (max_q_len < 1 || dims->total_q < 1 || (qo_indptr == nullptr && dims->q_len_fixed < 1)) return MLA_ERR_BAD_Q_LEN;
  ContractArgs c;
  c.block_tables = block_tables;
  c.seq_lens = seq_lens;
  c.qo_indptr = qo_indptr;
  c.result = result;
  c.num_pages = dims->num_pages;
  c.batch = dims->batch;
  c.bt_stride = dims->block_table_stride;
  c.page_size = dims->page_size;
  c.max_seq_len = max_seq_len;
  c.max_q_len = max_q_len;
  c.q_len_fixed = dims->q_len_fixed;
  c.total_q = dims->total_q;
  c.causal = causal != 0;
  hipLaunchKernelGGL(mla_check_contract_kernel, dim3(1), dim3(CHECK_THREADS), 0, (hipStream_t)stream, c);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

void mla_decode_internal_set_grid_override(int32_t grid) { g_grid_override.store(grid > 0 ? grid : 0); }

void mla_decode_internal_set_segment_cost(int32_t tiles) {
  g_seg_cost.store(tiles < 0 ? -1 : std::min(tiles, SEG_COST_MAX));
}

void mla_decode_internal_set_work_groups(int32_t enable) {
  g_groups.store(enable != 0 ? 1 : 0);
}

void mla_decode_internal_set_kernel_events(void* start_event, void* decode_event, void* stop_event) {
  g_ev_start.store(start_event);
  g_ev_decode.store(decode_event);
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
