// pagedkv.hip -- PagedAttention decode, split-K reduce and KV-write kernels for gfx950
// (AMD Instinct MI355X, CDNA4), behind the C ABI declared in include/pagedkv.h.
//
// What is computed is fixed by the pages: the KV cache is a pool of fixed-size blocks reached
// through a per-sequence block table ("vllm-project-vllm -- L2", section 3 Q2, section 6
// "KV Cache Block Tables"); decode reads the whole cache of every sequence for one new query
// token and is bound by memory bandwidth (same page, section 7).  How it is computed here is
// designed for CDNA4:
//
//  * Work unit = one wave (64 lanes) per KV head g over a stretch of tiles: a range of the
//    batch's (sequence, tile) stream (balanced split), one token partition, or one sequence.
//    The G query heads that share KV head g are the 16 columns of the MFMA tiles, so every
//    K/V byte is read from HBM once and used by all G heads.
//  * A tile is 16 consecutive tokens of one KV head, always inside one physical block (block
//    sizes are multiples of 16).  Scores S^T[16 tok x 16 head] = K[16 x D] . Q^T[D x 16] use
//    v_mfma_f32_16x16x32_{bf16,f16}; each lane loads its A-operand slice of K straight from
//    HBM with 16-byte loads.  Which physical d feeds which MFMA k-index is free (the sum over
//    d does not care), so loads are laid out for coalescing and q is loaded to match.
//  * Online softmax in the exp2 domain on the MFMA output layout: lane l holds 4 tokens of
//    head l%16, so the tile max needs two cross-lane steps and the running sum stays
//    lane-local until the end.  Tokens past the context are removed by select, never by
//    multiplying, and their K/V rows are read as zeros (the last tile's loads end at the
//    sequence's last row), so stale NaN bytes cannot leak in.
//  * O^T[D x 16 head] += V^T[D x 16 tok] . P^T[16 tok x 16 head] with v_mfma_f32_16x16x16.
//    V is staged through LDS in an XOR-swizzled layout and read back with gfx950's
//    ds_read_b64_tr_b16, which hands each lane 4 tokens of one d: exactly the operand layout.
//    Computing O^T (not O) keeps head = lane%16 in the accumulator, so the softmax rescale
//    factor is lane-local too.
//  * fp8 (OCP E4M3FN) caches are decoded to bf16/f16 in registers with
//    v_cvt_scalef32_pk_{bf16,f16}_fp8 (exact: every E4M3FN value is representable); the
//    per-tensor scales are folded into the softmax exponent and the output normalisation.
//  * The next tile's loads are issued before the current tile is computed.
//  * Split-K: partials (m, l, o) per partition, merged by paged_attn_reduce with log-sum-exp
//    weights.  Reduction orders are fixed, so results are deterministic.
//  * Shared prefix (pa_prefix_kernel): when every row starts with the same blocks, the prefix is
//    scored against many rows' queries at once -- a dense product on the matrix cores with K/V
//    stages in LDS -- and merged with each row's suffix partials from the decode above.
//  * Append (pa_decode_kernel<..., APPEND>): the step's new K/V row is used in place of the
//    stale pool row and stored into the pool by the wave that streams its tile, so the KV write
//    needs no launch of its own.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "pagedkv.h"
#include "host_util.h"

namespace {

using namespace pkv_host;

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef _Float16 f16x4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

enum { KF16 = PKV_F16, KBF16 = PKV_BF16, KFP8 = PKV_FP8_E4M3 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufWord3 = 0x00020000;   // gfx9 buffer descriptor word 3: 32-bit data format
// Cache policy of the K/V loads.  Private blocks are read exactly once per launch, so the loads
// are marked "nt" (non-temporal) and the caches are told not to keep them: measured 9-10%
// faster than the default policy on the Llama-3 decode batches (the scope bits sc0 / sc1 gave
// nothing or less).  When the caller says that physical blocks are shared by several rows
// (PKV_FLAG_SHARED_BLOCKS, e.g. a common prefix), the default policy keeps them in the
// Infinity Cache for the other readers.
constexpr int kStreamPolicy = 2;
constexpr int kCachedPolicy = 0;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ------------------------------------------------------------------ MFMA wrappers

template <bool BF>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <bool BF>
__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ conversions

// Two fp8 codes from the low (HI=false) or high 16 bits of w -> two 16-bit values, packed.
template <bool BF, bool HI>
__device__ __forceinline__ unsigned fp8x2_to_16(unsigned w) {
  if constexpr (BF)
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  else
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// 16 fp8 codes (one 16-byte load) -> 16 bf16/f16 values in two 16-byte registers.
template <bool BF>
__device__ __forceinline__ void fp8x16_to_16(u32x4 in, u32x4& lo, u32x4& hi) {
  lo.x = fp8x2_to_16<BF, false>(in.x);
  lo.y = fp8x2_to_16<BF, true>(in.x);
  lo.z = fp8x2_to_16<BF, false>(in.y);
  lo.w = fp8x2_to_16<BF, true>(in.y);
  hi.x = fp8x2_to_16<BF, false>(in.z);
  hi.y = fp8x2_to_16<BF, true>(in.z);
  hi.z = fp8x2_to_16<BF, false>(in.w);
  hi.w = fp8x2_to_16<BF, true>(in.w);
}

// A row of fp8 codes widened into LDS: the 16 codes of one 16-byte load become two 16-byte
// chunks (2c, 2c + 1) of 16-bit values.  A 16-byte store is serviced eight lanes (128 bytes of
// banks) at a time; if all eight stored their even chunk first, the chunk positions modulo 8
// would take only four values (the swizzles are even) and every store would conflict two ways.
// So lanes 4-7 of each group of eight (`flip`) store their odd chunk first: they swap the two
// input halves before widening, and the caller passes the two addresses in that order.  The
// layout and the reads are unchanged; only the order of the two stores differs between lanes.
__device__ __forceinline__ bool fp8_store_flip(int lane_or_index) { return ((lane_or_index >> 2) & 1) != 0; }

template <bool BF>
__device__ __forceinline__ void fp8x16_store_lds(u32x4 in, bool flip, char* first_slot, char* second_slot) {
  const u32x4 x = {flip ? in.z : in.x, flip ? in.w : in.y, flip ? in.x : in.z, flip ? in.y : in.w};
  u32x4 a, b;
  fp8x16_to_16<BF>(x, a, b);
  *(u32x4*)first_slot = a;
  *(u32x4*)second_slot = b;
}

template <bool BF>
__device__ __forceinline__ unsigned short f32_to_16(float x) {  // round to nearest even
  if constexpr (BF)
    return __builtin_bit_cast(unsigned short, (__bf16)x);
  else
    return __builtin_bit_cast(unsigned short, (_Float16)x);
}

template <bool BF>
__device__ __forceinline__ float from16(unsigned short h) {
  if constexpr (BF)
    return __uint_as_float((unsigned)h << 16);
  else
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ unsigned pack2(unsigned short lo, unsigned short hi) {
  return (unsigned)lo | ((unsigned)hi << 16);
}

// Two floats -> two 16-bit values (round to nearest even) packed lo | hi << 16, one
// v_cvt_pk_bf16_f32 for bf16.
template <bool BF>
__device__ __forceinline__ unsigned pack2_16(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  if constexpr (BF) {
    typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, b16x2));
  } else {
    typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, h16x2));
  }
}

// OCP E4M3FN code of y, nearest-even, saturating at +-448 (written from the format: bias 7,
// 3 mantissa bits, subnormals m * 2^-9, S.1111.111 = NaN, no infinities).
__device__ __forceinline__ unsigned e4m3fn_code(float y) {
  unsigned u = __float_as_uint(y);
  unsigned sign = (u >> 24) & 0x80u;
  unsigned a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;           // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;          // |y| >= 448, inf: saturate
  if (a < 0x3c800000u) {                              // |y| < 2^-6: multiples of 2^-9
    float t = __uint_as_float(a) * 512.0f;            // exact scaling by 2^9
    return sign | (unsigned)__builtin_rintf(t);       // ties to even; 8 -> 2^-6 (code 8)
  }
  // normal: keep 3 mantissa bits, round the 20 dropped bits to nearest even, rebias 127->7
  unsigned r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  return sign | (r - (120u << 3));
}

// ------------------------------------------------------------------ cross-lane helpers

// Butterfly partners across the four 16-lane rows, on the VALU (no LDS round trip):
// permlane16_swap pairs rows 0-1 and 2-3, permlane32_swap pairs the two 32-lane halves.  Both
// returned halves hold the same two operands, so op(r[0], r[1]) is the pair's combined value
// in every lane, bit for bit the same in both partners.
__device__ __forceinline__ float max_rows16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_rows32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_rows16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_rows32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the 64 lanes with DPP: shifts by 1, 2, 4, 8 inside each 16-lane
// row, then row 0's total into row 1 and row 2's into row 3 (row_bcast:15), then the first
// half's total into rows 2 and 3 (row_bcast:31).  Lanes without a source add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// ------------------------------------------------------------------ decode kernel

// Schedules: one workgroup per sequence; fixed token partitions; a balanced split of the
// batch's tile stream (both split schedules leave partials for paged_attn_reduce).
enum { MODE_SINGLE = 0, MODE_FIXED = 1, MODE_BALANCED = 2 };

// Balanced split: fewest tiles a workgroup gets (bounds the partial slots per sequence).
constexpr int kMinChunkTiles = 8;
// Waves (KV heads) per workgroup; grid.y covers further groups of KV heads.
constexpr int kMaxWaves = 8;

struct DecodeParams {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  const int32_t* lens;
  float* tmp_out;
  float* max_logits;
  float* exp_sums;
  const void* knew;  // append: the step's new K rows [B, Hkv, D], stored at position n - 1
  const void* vnew;  // append: the new V rows
  int B;
  int L;           // query tokens per sequence (1 for decode); MFMA columns = G * L
  int max_blocks;
  int Hq;
  int Hkv;
  int G;
  int BS;
  int num_blocks;
  int mode;
  int PS;          // fixed partitions: tokens per partition
  int Pslots;      // partial slots per (sequence, head) in the workspace
  int W;           // balanced: workgroups per head group
  int cap;         // context lengths are clamped to [0, cap] (cap = max_context_len, as in the reduce)
  int t0;          // balanced split: tiles skipped at the start of every sequence (a shared
                   // prefix handled elsewhere); the stream holds tiles [t0, ceil(n / 16))
  int slot0;       // partial slots below slot0 belong to someone else (the prefix pass)
  int compact;     // balanced split, partials in the compact layout: the overlap of sequence b with
                   // workgroup w is partial b + w (unique: overlaps are ordered in both b and w), so
                   // a row needs B + W - 1 slots, [B + W - 1][L * Hq] partials in all
  int tile_shift;  // log2(BS / 16)
  float c2;        // scale * k_scale * log2(e)
  float v_scale;
};

// Compile-time geometry of one 16-token tile for a wave of CT 16-column tiles.
template <int D, int KV, int CT = 1>
struct Tile {
  static constexpr int ESZ = (KV == KFP8) ? 1 : 2;         // bytes per cached element
  static constexpr int ROWB = D * ESZ;                      // bytes of one (token, head) row
  static constexpr int NS = D / 32;                         // QK k-steps (16x16x32)
  static constexpr int NT = D / 16;                         // PV d-tiles (16x16x16)
  static constexpr int KLD = (KV == KFP8) ? NS / 2 : NS;    // 16-byte K loads per lane
  static constexpr int CPRS = ROWB / 16;                    // 16-byte chunks per source row
  static constexpr int VLD = ROWB / 64;                     // 16-byte V loads per lane
  static constexpr int TPI = 64 / CPRS;                     // tokens covered by one V load
  static constexpr int CPR = D / 8;                         // 16-byte chunks per LDS row (16-bit)
  static constexpr int VLDS = 16 * D * 2;                   // the V tile
  static constexpr int QLDS = CT * NS * 64 * 16;            // one segment's q operands
  static constexpr int LDS_BYTES = VLDS + QLDS;             // per wave
  // Tiles in flight per wave.  An fp8 tile is half the bytes of a 16-bit one, so it keeps
  // two in flight to hold the same bytes per wave against the load latency.
  static constexpr int PF = (KV == KFP8) ? 2 : 1;
};

// LDS slot (16-byte unit) of chunk c of token row t; XOR swizzle spreads the transposed
// reads of 8 consecutive tokens over distinct bank groups.
template <int CPR>
__device__ __forceinline__ int lds_slot(int t, int c) {
  const int swz = (CPR == 16) ? ((2 * t) & 15) : (t & 6);
  return t * CPR + (c ^ swz);
}

__device__ __forceinline__ int clamp_len(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }
// Tiles of an n-token sequence past its first t0 tiles.
__device__ __forceinline__ int tiles_after(int n, int t0) {
  const int t = ((n + 15) >> 4) - t0;
  return t > 0 ? t : 0;
}
// Units the balanced split counts for such a sequence: one per tile, plus one in front of its
// first tile.  Every sequence a workgroup starts costs it a segment switch and a split-K partial
// (about one tile of streaming time, measured), so the extra unit keeps workgroups that start
// many short sequences from finishing last.
__device__ __forceinline__ int units_after(int n, int t0) {
  const int t = tiles_after(n, t0);
  return t > 0 ? t + 1 : 0;
}

// Balanced split of the batch's unit stream (units_after: each sequence is one unit followed
// by one unit per tile) of N units into Weff contiguous ranges whose sizes differ by at most
// one: the first `rem` ranges hold q+1 units, the rest q.  A workgroup processes the tiles
// whose units fall in its range.  Weff is the requested count, lowered so that
// q >= kMinChunkTiles.  32-bit arithmetic (N < 2^31 is checked on the host).
struct Split {
  int N, Weff, q, rem;
  Split() = default;
  __device__ __forceinline__ Split(int n_tiles, int W) {
    N = n_tiles;
    const int cap = N / kMinChunkTiles;
    Weff = W < cap ? W : cap;
    if (Weff < 1) Weff = 1;
    q = N / Weff;
    rem = N - q * Weff;
  }
  __device__ __forceinline__ int lo(int w) const { return w * q + (w < rem ? w : rem); }
  __device__ __forceinline__ int owner(int t) const {   // the range holding tile t
    const int big = rem * (q + 1);
    return t < big ? t / (q + 1) : rem + (t - big) / q;
  }
};

// A segment: tiles [tlo, thi) of sequence b (n tokens), written to partial `slot` (or, for
// slot < 0, as the final row).  All fields are wave-uniform.
struct Seg {
  int b, tlo, thi, n, slot;
  long long start;   // balanced split: global index of b's first tile
  bool valid;
};

// The ordered list of segments one workgroup processes.  For the balanced split the lengths
// and tile offsets of 64 consecutive sequences b0 .. b0+63 sit in two VGPRs (lane k holds
// sequence b0+k), so moving from one segment to the next is register work only; a workgroup
// whose range runs past b0+63 refills the table.
struct SegSource {
  int mode, B, cap, w, t0;
  Split split;
  long long lo, hi;
  const int32_t* lens;
  int b0;               // first sequence of the table
  long long base;       // global index of sequence b0's first tile
  int n_v, st_v;        // lane k: clamped length of b0+k, its first tile relative to base
  unsigned long long vmask;   // lanes whose sequence has a tile inside [lo, hi)

  __device__ __forceinline__ int len(int b) const {
    return clamp_len(__builtin_amdgcn_readfirstlane(lens[b]), cap);
  }
  // Table of sequences b .. b+63 given b's first unit; n_lane = len(b + lane) if already known.
  // st_v is the unit of the lane's first tile (past its sequence's leading unit).
  __device__ __forceinline__ void fill(int b, long long start, int lane, int n_lane) {
    b0 = b;
    base = start;
    n_v = n_lane;
    const int t = tiles_after(n_v, t0);
    st_v = wave_incl_scan(units_after(n_v, t0)) - t;
    const long long s0 = start + st_v;
    vmask = __ballot(t > 0 && s0 < hi && s0 + t > lo);
  }
  __device__ __forceinline__ void fill_load(int b, long long start, int lane) {
    const int bb = b + lane;
    fill(b, start, lane, bb < B ? clamp_len(lens[bb], cap) : 0);
  }
  __device__ __forceinline__ Seg make_lane(int k) const {
    Seg s;
    s.b = b0 + k;
    s.n = __builtin_amdgcn_readlane(n_v, k);
    s.start = base + __builtin_amdgcn_readlane(st_v, k);
    const long long nt = tiles_after(s.n, t0);
    const long long a = lo > s.start ? lo : s.start;
    const long long e = hi < s.start + nt ? hi : s.start + nt;
    s.tlo = t0 + (int)(a - s.start);                    // tile numbers within the sequence
    s.thi = t0 + (int)(e - s.start);
    s.slot = w - split.owner((int)s.start);
    s.valid = true;
    return s;
  }
  // The first segment at or after table lane k, refilling the table past its end.
  __device__ __forceinline__ Seg from_lane(int k, int lane) {
    for (;;) {
      const unsigned long long m = k < 64 ? (vmask >> k) << k : 0ull;
      if (m) return make_lane(__builtin_ctzll(m));
      // nothing left in this table: does the range continue past sequence b0+63?
      const int n63 = __builtin_amdgcn_readlane(n_v, 63);
      const long long next_start = base + __builtin_amdgcn_readlane(st_v, 63) + tiles_after(n63, t0);
      if (b0 + 64 >= B || next_start >= hi) {
        Seg r;
        r.valid = false;
        return r;
      }
      fill_load(b0 + 64, next_start, lane);
      k = 0;
    }
  }
  // The segment after s (balanced split only; the other schedules have one segment).
  __device__ __forceinline__ Seg next(const Seg& s, int lane) {
    Seg r;
    r.valid = false;
    if (mode != MODE_BALANCED) return r;
    return from_lane(s.b - b0 + 1, lane);
  }
};

// Balanced split, the first segment of workgroup w out of W: every wave of the workgroup runs
// this with the same result.  Scans the lengths (units_after: one unit per tile past t0, plus one
// per sequence), cuts the unit stream into W ranges and positions `src` at the first sequence
// of range w.  Returns false when the range holds no tile.
__device__ __forceinline__ bool balanced_start(SegSource& src, Seg& cur, const int32_t* lens, int B, int cap,
                                               int t0, int W, int w, int lane) {
  src.mode = MODE_BALANCED;
  src.B = B;
  src.cap = cap;
  src.lens = lens;
  src.t0 = t0;
  const int per = (B + 63) >> 6;                        // sequences per lane in the scan
  int run = 0, n_first = 0;
  for (int i = 0; i < per; ++i) {
    const int bb = lane * per + i;
    const int n = bb < B ? clamp_len(lens[bb], cap) : 0;
    if (i == 0) n_first = n;
    run += units_after(n, t0);
  }
  const int incl = wave_incl_scan(run);                 // inclusive scan over lanes
  const int N = __builtin_amdgcn_readlane(incl, 63);
  if (N == 0) return false;
  const Split split(N, W);
  if (w >= split.Weff) return false;
  src.w = w;
  src.split = split;
  src.lo = split.lo(w);
  src.hi = split.lo(w + 1);
  if (per == 1) {
    src.fill(0, 0, lane, n_first);                      // the scan already holds every length
  } else {
    // the lane whose run of sequences holds tile `lo` starts the table
    const unsigned long long hit = __ballot(incl > src.lo);
    if (hit == 0) return false;                         // unreachable for lo < N
    const int L = __builtin_ctzll(hit);
    src.fill_load(L * per, __builtin_amdgcn_readlane(incl - run, L), lane);
  }
  cur = src.from_lane(0, lane);
  return cur.valid;
}

// One workgroup = up to kMaxWaves waves; wave i handles KV head g = blockIdx.y*kMaxWaves + i,
// so the waves stream whole blocks ([BS][Hkv][D] is contiguous) together.  Each wave owns one
// LDS tile and runs one continuous tile pipeline over all segments of its workgroup: the next
// tile's loads go out while the current tile is computed, also across segment boundaries.
// Every load result is first read at least one tile after it was issued, and nothing waits
// on a value right after loading it, so the in-order load counter never drains the tile
// in flight.
//
// APPEND (16-bit caches): the step's new token of every sequence is not in the pool yet.  The
// wave that streams the tile holding position n - 1 fetches the new K/V row of its head
// together with that tile's loads, uses it in place of the stale pool row and stores it into
// the pool; no other workgroup reads that slot during the launch.
//
// CT > 1 (multi-query with 17 .. 16 * CT (head, new token) columns per KV group): each wave carries
// CT tiles of 16 MFMA columns; every K and V operand it loads feeds all CT tiles.
template <int D, int KV, bool BF, int MODE, int POLICY, bool APPEND = false, int CT = 1>
__global__ __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(2)))
void pa_decode_kernel(DecodeParams a) {
  using TL = Tile<D, KV, CT>;
  static_assert(!APPEND || (KV != KFP8 && TL::PF == 1 && CT == 1), "append is for 16-bit caches, one tile in flight");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int wl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.y * kMaxWaves + wl;               // KV head of this wave
  if (g >= a.Hkv) return;
  char* vtile = smem + wl * TL::LDS_BYTES;
  char* qstage = vtile + TL::VLDS;                          // next segment's q, lane-major
  const int cap = a.cap;

  // ---- the workgroup's segments
  SegSource src;
  src.mode = MODE;
  src.B = a.B;
  src.cap = cap;
  src.lens = a.lens;
  src.w = 0;
  src.t0 = MODE == MODE_BALANCED ? a.t0 : 0;
  src.split = Split(1, 1);
  src.lo = 0;
  src.hi = 0;
  Seg cur;
  if constexpr (MODE == MODE_SINGLE) {
    cur.b = blockIdx.x;
    cur.n = src.len(cur.b);
    cur.tlo = 0;
    cur.thi = (cur.n + 15) >> 4;
    cur.slot = -1;
    cur.start = 0;
    cur.valid = true;
  } else if constexpr (MODE == MODE_FIXED) {
    cur.b = blockIdx.z;
    cur.n = src.len(cur.b);
    cur.slot = blockIdx.x;
    cur.tlo = (cur.slot * a.PS) >> 4;
    cur.thi = (min((cur.slot + 1) * a.PS, cur.n) + 15) >> 4;
    cur.start = 0;
    cur.valid = cur.thi > cur.tlo;
    if (!cur.valid) return;
  } else {
    // MODE_BALANCED: equal contiguous ranges of the batch's (sequence, tile) stream
    if (!balanced_start(src, cur, a.lens, a.B, cap, src.t0, a.W, blockIdx.x, lane)) return;
  }
  // Issue priority by progress (balanced split: every wave of the workgroup streams the same
  // tiles of its own head).  The sequencer favours a SIMD's older wave, so with equal priority
  // the first wave on each SIMD (waves 0-3 of a full workgroup) runs ahead and the second
  // (waves 4-7, on the same SIMDs) finishes ~6% of the launch later.
  //  - 16-bit caches, 8-wave workgroups: each wave publishes its tile count in LDS and compares
  //    it with its SIMD partner's (wave wl ^ 4) every tile; the wave that is ahead drops to the
  //    lowest priority, the one behind takes the highest.  The pair stays within a tile.
  //  - otherwise (fp8 caches, whose widening keeps the SIMD busy and gains from one wave running
  //    ahead; workgroups of fewer waves; a last head group whose partner wave has no head):
  //    each wave starts at the highest level and steps down a level per quarter of its tiles.
  // Priorities only order instruction issue; no result depends on them.
  int prog = 0, pq1 = 0, pq2 = 0, pq3 = 0;
  __shared__ int progs[kMaxWaves];                      // tiles started, per wave
  const bool pairs = MODE == MODE_BALANCED && KV != KFP8 && (blockDim.x >> 6) == kMaxWaves &&
                     blockIdx.y * kMaxWaves + (wl ^ 4) < a.Hkv;   // the partner has a head
  if constexpr (MODE == MODE_BALANCED) {
    const int tot = (int)(src.hi - src.lo);
    pq1 = tot >> 2;
    pq2 = tot >> 1;
    pq3 = tot - (tot >> 2);
    if (pairs) {
      __hip_atomic_store(&progs[wl], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __builtin_amdgcn_s_setprio(1);
    } else {
      __builtin_amdgcn_s_setprio(3);
    }
  }

  // ---- per-lane constants
  // MFMA column hh = (query head hh / L of the group, new query token hh % L).  Token i of the
  // L new tokens sits at position n - L + i and sees the first n - (L - 1 - i) tokens.
  // Tile c holds columns 16 c .. 16 c + 15.
  const int hh = lane & 15;
  const int grp = lane >> 4;    // MFMA row group
  bool hvalid[CT];
  int qi[CT], hoff[CT], hidden[CT];                     // hidden: newer tokens the column must not see
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    hvalid[c] = 16 * c + hh < a.G * a.L;
    const int hsel = hvalid[c] ? 16 * c + hh : 0;
    qi[c] = hsel % a.L;
    hoff[c] = g * a.G + hsel / a.L;
    hidden[c] = a.L - 1 - qi[c];
  }
  const int rowstride = a.Hkv * TL::ROWB;               // bytes between consecutive tokens
  int koff[TL::KLD];
#pragma unroll
  for (int i = 0; i < TL::KLD; ++i) koff[i] = (lane & 15) * rowstride + (4 * i + grp) * 16;
  int voff[TL::VLD];
  int vslot[TL::VLD];    // LDS byte offset of the (first) 16-bit chunk this load fills
  int vslot2[TL::VLD];   // fp8 only: the second chunk (16 codes widen to 32 bytes)
  const bool vflip = fp8_store_flip(lane);              // fp8: store order of the widened chunks
#pragma unroll
  for (int r = 0; r < TL::VLD; ++r) {
    const int t = r * TL::TPI + lane / TL::CPRS;
    const int cs = lane % TL::CPRS;
    voff[r] = t * rowstride + cs * 16;
    if constexpr (KV == KFP8) {
      // stored in this order (see fp8x16_store_lds)
      vslot[r] = lds_slot<TL::CPR>(t, 2 * cs + (vflip ? 1 : 0)) * 16;
      vslot2[r] = lds_slot<TL::CPR>(t, 2 * cs + (vflip ? 0 : 1)) * 16;
    } else {
      vslot[r] = lds_slot<TL::CPR>(t, cs) * 16;
      vslot2[r] = 0;
    }
  }
  int troff[TL::NT];
  {
    const int tt = 4 * grp + ((lane >> 2) & 3);
    const int qq = lane & 3;
#pragma unroll
    for (int T = 0; T < TL::NT; ++T)
      troff[T] = lds_slot<TL::CPR>(tt, 2 * T + (qq >> 1)) * 16 + (qq & 1) * 8;
  }
  const char* kbase = (const char*)a.kc + (size_t)g * TL::ROWB;
  const char* vbase = (const char*)a.vc + (size_t)g * TL::ROWB;
  const size_t blockbytes = (size_t)a.BS * rowstride;
  const int tshift = a.tile_shift;                      // log2(BS / 16)
  const int tmask = (1 << tshift) - 1;
  const unsigned nbm1 = (unsigned)(a.num_blocks - 1);
  const int tile_span = 15 * rowstride + TL::ROWB;

  // q of sequence b as the B operand of S^T = K . Q^T, d order matching the K loads.  Lanes
  // of MFMA columns >= G load a valid head of the group: those columns are computed and
  // dropped, and no select on the loaded value forces a wait right after the loads.
  auto load_q = [&](int b, u32x4 (*qv)[TL::NS]) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const char* qrow = (const char*)a.q + (((size_t)b * a.L + qi[c]) * a.Hq + hoff[c]) * D * 2;
#pragma unroll
      for (int s = 0; s < TL::NS; ++s) {
        int d0;
        if constexpr (KV == KFP8)
          d0 = 64 * (s >> 1) + 16 * grp + 8 * (s & 1);
        else
          d0 = 32 * s + 8 * grp;
        qv[c][s] = *(const u32x4*)(qrow + d0 * 2);
      }
    }
  };
  // Physical block of logical tile `tile` of sequence b (a wave-uniform address).  A valid
  // length keeps the entry index below ceil(n / BS) <= max_blocks; a length past the table only
  // re-reads the row's last entry, so it spoils that sequence's result alone and never leaves
  // the table.
  const int lastcol = a.max_blocks - 1;
  auto load_id = [&](int b, int tile) -> int {
    return a.bt[(size_t)b * a.max_blocks + min(tile >> tshift, lastcol)];
  };
  // Raw buffer loads: the descriptor base is the tile's first row (scalar), the lane offsets
  // are fixed VGPRs, and the descriptor's range covers exactly the tile's rows of head g
  // (span bytes; a span of 0 puts every lane out of range: the loads return zeros without
  // touching memory).  Block ids outside [0, num_blocks) are clamped so no access leaves the
  // pool.
  auto load_tile = [&](unsigned id, int tile, u32x4* kd, u32x4* vd, int span) {
    const size_t off = (size_t)min(id, nbm1) * blockbytes + (size_t)(tile & tmask) * 16 * rowstride;
    const __amdgpu_buffer_rsrc_t kres =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + off), (short)0, span, kBufWord3);
    const __amdgpu_buffer_rsrc_t vres =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + off), (short)0, span, kBufWord3);
#pragma unroll
    for (int i = 0; i < TL::KLD; ++i)
      kd[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, koff[i], 0, POLICY));
#pragma unroll
    for (int r = 0; r < TL::VLD; ++r)
      vd[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, voff[r], 0, POLICY));
  };

  // ---- softmax / accumulator state of the current segment
  f32x4 acc[CT][TL::NT];
  float m[CT], lsum[CT];
  auto reset = [&]() {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
#pragma unroll
      for (int T = 0; T < TL::NT; ++T) acc[c][T] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[c] = -INFINITY;
      lsum[c] = 0.f;
    }
  };
  reset();

  // First half of a tile: scores S^T = K . Q^T and the V tile into LDS.  After it the tile's
  // registers are free, so the next tile's loads can land in them.  Rows >= n of a sequence's
  // last tile arrive as zeros (their loads are out of the tile's buffer range), so stale bytes,
  // which may be NaN, never reach the scores or the V tile.
  auto part1 = [&](const u32x4* kr, const u32x4* vr, const u32x4 (*qv)[TL::NS], f32x4* s) {
#pragma unroll
    for (int c = 0; c < CT; ++c) s[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < TL::NS; ++st) {
      u32x4 kop;
      if constexpr (KV == KFP8) {
        u32x4 lo, hi;
        fp8x16_to_16<BF>(kr[st >> 1], lo, hi);
        kop = (st & 1) ? hi : lo;
      } else {
        kop = kr[st];
      }
#pragma unroll
      for (int c = 0; c < CT; ++c) s[c] = mfma_16x16x32<BF>(kop, qv[c][st], s[c]);
    }
#pragma unroll
    for (int r = 0; r < TL::VLD; ++r) {
      if constexpr (KV == KFP8)
        fp8x16_store_lds<BF>(vr[r], vflip, vtile + vslot[r], vtile + vslot2[r]);
      else
        *(u32x4*)(vtile + vslot[r]) = vr[r];
    }
  };

  // Second half: online softmax (exp2 domain) and O^T += V^T . P^T.  Tokens a column may not
  // see (>= n, or newer than its own query token) are selected out of the scores; a tile that
  // every column sees whole (all but the last tile or two of a segment) skips the selects.  A
  // column that has seen no token yet keeps m = -inf; its probabilities are computed against
  // 0 so that they come out 0, not NaN.
  auto part2 = [&](int tile, int n, const f32x4* s) {
    const int tbase = (tile << 4) + 4 * grp;
    const bool whole = ((tile + 1) << 4) <= n - (a.L - 1);   // every column sees the whole tile
    u32x2 pop[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      float x[4];
      if (whole) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = s[c][e] * a.c2;
      } else {
        const int lim = n - hidden[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (tbase + e < lim) ? s[c][e] * a.c2 : -INFINITY;
      }
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = max_rows32(max_rows16(mx));
      if (__ballot(mx > m[c]) != 0) {
        // every lane rescales when any column's maximum rises; a column that has seen no token
        // yet (m = -inf, possible under the causal mask) has nothing to rescale
        const float mn = fmaxf(m[c], mx);
        const float alpha = m[c] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[c] - mn);
        m[c] = mn;
        lsum[c] *= alpha;
#pragma unroll
        for (int T = 0; T < TL::NT; ++T) acc[c][T] *= alpha;
      }
      unsigned short ph[4];
      const float mb = m[c] == -INFINITY ? 0.f : m[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ph[e] = f32_to_16<BF>(__builtin_amdgcn_exp2f(x[e] - mb));
        lsum[c] += from16<BF>(ph[e]);
      }
      pop[c] = u32x2{pack2(ph[0], ph[1]), pack2(ph[2], ph[3])};
    }
#pragma unroll
    for (int T = 0; T < TL::NT; ++T) {
      s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_char*)vtile + troff[T]));
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[c][T] = mfma_16x16x16<BF>(__builtin_bit_cast(u32x2, raw), pop[c], acc[c][T]);
    }
  };

  // Total sum over the 4 row groups, normalise, store the row or the partial.
  auto finalize = [&](const Seg& sg) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const float l = sum_rows32(sum_rows16(lsum[c]));
      const float inv = l > 0.f ? a.v_scale / l : 0.f;
      if (!hvalid[c]) continue;
      if constexpr (MODE == MODE_SINGLE) {
        unsigned short* orow = (unsigned short*)a.out + (((size_t)sg.b * a.L + qi[c]) * a.Hq + hoff[c]) * D;
#pragma unroll
        for (int T = 0; T < TL::NT; ++T) {
          u32x2 wv;
          wv.x = pack2(f32_to_16<BF>(acc[c][T][0] * inv), f32_to_16<BF>(acc[c][T][1] * inv));
          wv.y = pack2(f32_to_16<BF>(acc[c][T][2] * inv), f32_to_16<BF>(acc[c][T][3] * inv));
          *(u32x2*)(orow + 16 * T + 4 * grp) = wv;
        }
      } else if (sg.slot >= 0 && (a.compact || a.slot0 + sg.slot < a.Pslots)) {
        const size_t prow = a.compact ? (size_t)(sg.b + src.w) * a.L * a.Hq + (size_t)qi[c] * a.Hq + hoff[c]
                                      : (((size_t)sg.b * a.L + qi[c]) * a.Hq + hoff[c]) * a.Pslots + a.slot0 + sg.slot;
        float* orow = a.tmp_out + prow * D;
#pragma unroll
        for (int T = 0; T < TL::NT; ++T) *(f32x4*)(orow + 16 * T + 4 * grp) = acc[c][T] * inv;
        if (grp == 0) {
          a.max_logits[prow] = m[c] * kLn2;
          a.exp_sums[prow] = l;
        }
      }
    }
  };

  if (cur.thi <= cur.tlo) {                             // single pass, empty context: zeros
    finalize(cur);
    return;
  }

  // ---- prologue: q of the first segment, the first tile's block id and the first tiles.
  // The next segment's q goes through LDS: loaded into qn at a segment switch, written to the
  // wave's LDS stage one tile later (when the load has landed, so the write does not drain
  // the tiles in flight), and read back into qc at the next switch.  Registers loaded from
  // memory are never copied, which would force a wait right after the load.
  Seg nxt = src.next(cur, lane);
  u32x4 qc[CT][TL::NS], qn[CT][TL::NS];
  load_q(cur.b, qc);
  bool qpend = nxt.valid;
  if (qpend) load_q(nxt.b, qn);

  // Issue iterator: (iseg, itile) is the next tile to load; its block id sits in `nid`,
  // loaded one tile ahead of the tile's own loads, so reading it never waits for loads that
  // are still in flight.
  SegSource isrc = src;                                 // own table: the iterators run
  Seg iseg = cur;                                       // at different positions
  int itile = cur.tlo;
  bool idone = false;
  int nid = load_id(cur.b, cur.tlo);
  // Load the tile at the issue position, then advance it and fetch the next block id.  The
  // range ends at the sequence's last row, so rows >= n of its last tile read as zeros.  Past
  // the stream's end the same load instructions go out with an empty range (zeros, no memory
  // traffic), which keeps every load unconditional: a skipped load would make the compiler
  // wait for every load in flight before the next tile.
  // Append state of the tile in flight: whether it holds the new token, the token's row in the
  // tile, the pool offset of that row (head g), and the new row's values for the lanes that
  // hold it in the A operand (K) and in the V load pattern.
  bool apn = false;
  int aprow = 0;
  size_t apoff = 0;
  u32x4 knew[APPEND ? TL::KLD : 1], vnew;
  auto issue = [&](u32x4* kd, u32x4* vd) {
    const unsigned id = (unsigned)__builtin_amdgcn_readfirstlane(nid);
    const int rows = iseg.n - (itile << 4);             // rows of the tile below n (>= 1)
    load_tile(id, itile, kd, vd, idone ? 0 : (rows >= 16 ? tile_span : (rows - 1) * rowstride + TL::ROWB));
    if constexpr (APPEND) {
      apn = !idone && itile == ((iseg.n - 1) >> 4);
      if (apn) {
        aprow = (iseg.n - 1) & 15;
        apoff = (size_t)min(id, nbm1) * blockbytes + (size_t)((iseg.n - 1) & (a.BS - 1)) * rowstride;
        const size_t roff = ((size_t)iseg.b * a.Hkv + g) * TL::ROWB;
        if ((lane & 15) == aprow) {
#pragma unroll
          for (int i = 0; i < TL::KLD; ++i)
            knew[i] = *(const u32x4*)((const char*)a.knew + roff + (4 * i + grp) * 16);
        }
        if (lane / TL::CPRS == aprow % TL::TPI)
          vnew = *(const u32x4*)((const char*)a.vnew + roff + (lane % TL::CPRS) * 16);
      }
    }
    if (idone) return;
    if (itile + 1 < iseg.thi) {
      ++itile;
    } else {
      const Seg s2 = isrc.next(iseg, lane);
      if (!s2.valid) {
        idone = true;
        return;
      }
      iseg = s2;
      itile = s2.tlo;
    }
    nid = load_id(iseg.b, itile);
  };

  // PF register sets of K/V rows rotate through the loop: set r is computed, then refilled
  // with the tile PF positions ahead, so PF tiles stay in flight per wave.
  u32x4 kr[TL::PF][TL::KLD], vr[TL::PF][TL::VLD];
#pragma unroll
  for (int r = 0; r < TL::PF; ++r) issue(kr[r], vr[r]);

  int tile = cur.tlo;
  bool done = false;
  while (!done) {
#pragma unroll
    for (int r = 0; r < TL::PF; ++r) {
      if constexpr (MODE == MODE_BALANCED) {
        if (pairs) {
          __hip_atomic_store(&progs[wl], prog, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          const int d = prog - __builtin_amdgcn_readfirstlane(
                                   __hip_atomic_load(&progs[wl ^ 4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
          if (d > 0)
            __builtin_amdgcn_s_setprio(0);
          else if (d < 0)
            __builtin_amdgcn_s_setprio(3);
          else
            __builtin_amdgcn_s_setprio(1);
        } else {
          if (prog == pq1) __builtin_amdgcn_s_setprio(2);
          if (prog == pq2) __builtin_amdgcn_s_setprio(1);
          if (prog == pq3) __builtin_amdgcn_s_setprio(0);
        }
        ++prog;
      }
      if constexpr (APPEND) {
        if (apn) {                                      // this tile holds the new token
          const bool kl = (lane & 15) == aprow;
          const bool vl = lane / TL::CPRS == aprow % TL::TPI;
#pragma unroll
          for (int i = 0; i < TL::KLD; ++i) kr[r][i] = kl ? knew[i] : kr[r][i];
#pragma unroll
          for (int j = 0; j < TL::VLD; ++j) vr[r][j] = (vl && j == aprow / TL::TPI) ? vnew : vr[r][j];
          if (kl) {
#pragma unroll
            for (int i = 0; i < TL::KLD; ++i) *(u32x4*)((char*)kbase + apoff + (4 * i + grp) * 16) = knew[i];
          }
          if (vl) *(u32x4*)((char*)vbase + apoff + (lane % TL::CPRS) * 16) = vnew;
        }
      }
      f32x4 sc[CT];
      part1(kr[r], vr[r], qc, sc);
      __builtin_amdgcn_sched_barrier(0);
      issue(kr[r], vr[r]);                              // set r is free again
      __builtin_amdgcn_sched_barrier(0);
      part2(tile, cur.n, sc);
      if (qpend) {
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int s = 0; s < TL::NS; ++s) *(u32x4*)(qstage + ((c * TL::NS + s) * 64 + lane) * 16) = qn[c][s];
        qpend = false;
      }
      if (tile + 1 < cur.thi) {
        ++tile;
        continue;
      }
      finalize(cur);
      if (!nxt.valid) {
        done = true;
        break;
      }
      // next segment: its q is in the LDS stage; the q of the one after it is loaded now
      reset();
      cur = nxt;
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int s = 0; s < TL::NS; ++s) qc[c][s] = *(const u32x4*)(qstage + ((c * TL::NS + s) * 64 + lane) * 16);
      nxt = src.next(cur, lane);
      qpend = nxt.valid;
      if (qpend) load_q(nxt.b, qn);
      tile = cur.tlo;
    }
  }
}

// ------------------------------------------------------------------ tiled passes

// Two passes score MANY query columns against one KV head's tokens, which makes them dense
// contractions on the matrix cores rather than streams:
//  * the shared-prefix pass: when every row of a batch starts with the same blocks (shared
//    copy-on-write), the decode above would stream the prefix once per row.  Here it is read
//    once per workgroup and scored against many rows' queries together: for KV head g,
//    S = Q_g . K_prefix^T over all B * G query rows of that head;
//  * multi-query attention with many new tokens per sequence (chunked prefill, long draft
//    verification): for sequence b and KV head g the G * L (head, new token) pairs are the
//    columns, each with its own causal limit.
// Both share one core.  A workgroup of NW waves takes one KV head, a block of NW * CT * 16
// columns and a token range.  64-token stages of K and V pass through LDS once for all waves
// (fp8 is widened to 16 bits on the way in), double-buffered, so the next stage's global loads
// fly while the current one is computed.  Each wave owns CT tiles of 16 columns and runs their
// online softmax; QK^T and PV both use v_mfma_f32_16x16x32, and each K or V operand read from
// LDS feeds all CT column tiles of the wave.

constexpr int kStage = 64;                       // tokens per LDS stage

template <int D, int KV>
struct StageGeom {
  static constexpr int ESZ = (KV == KFP8) ? 1 : 2;
  static constexpr int ROWB = D * ESZ;                          // source bytes per (token, head)
  static constexpr int CPRS = ROWB / 16;                        // 16-byte source chunks per row
  static constexpr int CPR = D / 8;                             // 16-byte chunks of a 16-bit row
  static constexpr int NCH = kStage * CPRS;                     // source chunks per stage and pool
  static constexpr int KST = kStage * D * 2;                    // one pool's stage in LDS
  static constexpr int SUB = 16 * D * 2;                        // a 16-token sub-tile
  static constexpr int STAGE = 2 * KST;                         // K, then V
  static constexpr int LDS_BYTES = 2 * STAGE;                   // double-buffered: 64 KiB at D = 128
  static constexpr int NS = D / 32;
  static constexpr int NT = D / 16;
};

// Where a pass's stage rows come from: KV head g of both pools, through one block-table row.
struct StageSrc {
  const char* kc;          // K pool, advanced to head g
  const char* vc;
  const int32_t* row;      // the block-table row
  int rowstride;           // bytes between consecutive tokens of a block
  size_t blockbytes;
  int bs_shift;            // log2(block_size)
  int lastcol;             // last entry of the row (indices are clamped to it)
  unsigned nbm1;           // num_blocks - 1 (ids are clamped to it)
};

// K rows in LDS: chunk c of row t sits at c ^ swizzle(t), so the 16 rows that one MFMA
// A-operand read touches (16 lanes, same logical chunk) land in 16 distinct bank groups.
template <int CPR>
__device__ __forceinline__ int kslot(int t, int c) {
  const int swz = (CPR == 16) ? (t & 15) : ((t >> 1) & 7);
  return t * CPR + (c ^ swz);
}

// The workgroup's stage pipeline: thread tid moves source chunks tid, tid + 64 * NW, ... of K
// and of V.  Rows at or past `tend` are zero in LDS.  The block ids of a stage's rows are
// loaded one stage before its K/V rows, so the row loads never wait on them.
// Load k of a wave covers chunks 64 * (wave + k * NW) .. + 63, i.e. 64 / CPRS consecutive tokens
// (4, 8 or 16).  Stage starts are multiples of 16 tokens, so those tokens lie in one 16-token
// tile and hence in one block: the row address and the buffer range of a K/V load are
// wave-uniform (scalar), and each lane adds a fixed offset.  (The ids stay per-lane loads: a
// scalar id load measured slower in the shared-prefix pass.)
template <int D, int KV, bool BF, int NW>
struct Stages {
  using SG = StageGeom<D, KV>;
  static constexpr int NLD = (SG::NCH + 64 * NW - 1) / (64 * NW);
  static constexpr int TPW = 64 / SG::CPRS;                     // tokens per wave and load
  u32x4 kreg[NLD], vreg[NLD];
  int idn[NLD];

  __device__ __forceinline__ void load_ids(const StageSrc& s, int tid, int tok0, int tend) {
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int ci = tid + k * 64 * NW;
      const int tok = tok0 + ci / SG::CPRS;
      idn[k] = (ci < SG::NCH && tok < tend) ? s.row[min(tok >> s.bs_shift, s.lastcol)] : 0;
    }
  }
  __device__ __forceinline__ void load(const StageSrc& s, int tid, int tok0, int tend) {
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int loff = (lane / SG::CPRS) * s.rowstride + (lane % SG::CPRS) * 16;
    const int bsm1 = (1 << s.bs_shift) - 1;
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int ci0 = 64 * (wv + k * NW);
      if (ci0 >= SG::NCH) {                                     // no chunk of this load (wave-uniform)
        kreg[k] = u32x4{0u, 0u, 0u, 0u};
        vreg[k] = u32x4{0u, 0u, 0u, 0u};
        continue;
      }
      const int tok = tok0 + ci0 / SG::CPRS;
      const int nt = tend - tok;                                // tokens of this load below tend
      // the range ends at the last valid token's row: lanes past it read zeros, no memory access
      const int span = nt <= 0 ? 0 : (min(nt, TPW) - 1) * s.rowstride + SG::ROWB;
      const unsigned id = min((unsigned)__builtin_amdgcn_readfirstlane(idn[k]), s.nbm1);
      const size_t off = (size_t)id * s.blockbytes + (size_t)(tok & bsm1) * s.rowstride;
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(s.kc + off), (short)0, span, kBufWord3);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(s.vc + off), (short)0, span, kBufWord3);
      kreg[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, loff, 0, kCachedPolicy));
      vreg[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, loff, 0, kCachedPolicy));
    }
  }
  __device__ __forceinline__ void store(char* st, int tid) {
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int ci = tid + k * 64 * NW;
      if (ci >= SG::NCH) continue;
      const int t = ci / SG::CPRS, cs = ci % SG::CPRS;
      char* vst = st + SG::KST + (t >> 4) * SG::SUB;
      if constexpr (KV == KFP8) {
        const bool f = fp8_store_flip(ci);                      // ci and the lane agree modulo 8
        const int c1 = 2 * cs + (f ? 1 : 0), c2 = 2 * cs + (f ? 0 : 1);
        fp8x16_store_lds<BF>(kreg[k], f, st + kslot<SG::CPR>(t, c1) * 16, st + kslot<SG::CPR>(t, c2) * 16);
        fp8x16_store_lds<BF>(vreg[k], f, vst + lds_slot<SG::CPR>(t & 15, c1) * 16,
                             vst + lds_slot<SG::CPR>(t & 15, c2) * 16);
      } else {
        *(u32x4*)(st + kslot<SG::CPR>(t, cs) * 16) = kreg[k];
        *(u32x4*)(vst + lds_slot<SG::CPR>(t & 15, cs) * 16) = vreg[k];
      }
    }
  }
};

// One wave's CT tiles of 16 query columns: q operands, per-column limits and the online
// softmax state.  Lane l holds column l % 16 of every tile; the column sees the tokens below
// its limit.  O^T and the softmax row sums accumulate on the matrix cores.
template <int D, bool BF, int CT>
struct ColTiles {
  static constexpr int NS = D / 32, NT = D / 16, KST = kStage * D * 2, SUB = 16 * D * 2, CPR = D / 8;
  u32x4 qv[CT][NS];
  f32x4 acc[CT][NT];
  f32x4 accL[CT];      // every element: the column's running sum of probabilities
  float m[CT];         // running maximum (exp2 domain); -inf until the column sees a token
  int lim[CT];         // this lane's column limit, per tile
  int wmin, wlim;      // lowest / highest limit over the wave's columns (wave-uniform)
  int koff[NS], troff[NT];
  int grp;

  __device__ __forceinline__ void init(int lane) {
    grp = lane >> 4;
#pragma unroll
    for (int s = 0; s < NS; ++s) koff[s] = kslot<CPR>(lane & 15, 4 * s + grp) * 16;
    const int tt = 4 * grp + ((lane >> 2) & 3);
    const int qq = lane & 3;
#pragma unroll
    for (int T = 0; T < NT; ++T) troff[T] = lds_slot<CPR>(tt, 2 * T + (qq >> 1)) * 16 + (qq & 1) * 8;
  }
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
#pragma unroll
      for (int T = 0; T < NT; ++T) acc[c][T] = f32x4{0.f, 0.f, 0.f, 0.f};
      accL[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[c] = -INFINITY;
    }
  }
  // q row of tile c (d order matching the K operand reads).
  __device__ __forceinline__ void load_q(int c, const char* qrow) {
#pragma unroll
    for (int s = 0; s < NS; ++s) qv[c][s] = *(const u32x4*)(qrow + (32 * s + 8 * grp) * 2);
  }
  // After setting lim[]: the wave's lowest and highest limits.
  __device__ __forceinline__ void limits_done() {
    int lo = lim[0], hi = lim[0];
#pragma unroll
    for (int c = 1; c < CT; ++c) {
      lo = min(lo, lim[c]);
      hi = max(hi, lim[c]);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      lo = min(lo, __shfl_xor(lo, o));
      hi = max(hi, __shfl_xor(hi, o));
    }
    wmin = __builtin_amdgcn_readfirstlane(lo);
    wlim = __builtin_amdgcn_readfirstlane(hi);
  }

  // One stage for the wave's columns: S^T of four 16-token sub-tiles per column tile, one
  // softmax update over all 64 tokens, then O^T += V^T . P^T two sub-tiles at a time.  MASKED:
  // some column of the wave stops inside the stage (per-column select on the scores, zeroed V
  // rows past every column's limit); otherwise the exponent is one fma per score.
  template <bool MASKED>
  __device__ __forceinline__ void compute(const char* st, int tok0, float c2) {
    // Every LDS operand of the stage's QK^T, and the V operands of the first PV half, is
    // requested before the first MFMA; the second half's V reads go out before the softmax.
    // LDS reads of a wave return in order, so each MFMA waits only for its own operand and
    // the LDS latency is paid about once per stage instead of once per MFMA.
    const char* vst = st + KST;
    auto vread = [&](int sub, int T) {
      return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)((lds_char*)(vst + sub * SUB) + troff[T])));
    };
    u32x4 kf[4][NS];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int s = 0; s < NS; ++s) kf[u][s] = *(const u32x4*)(st + u * SUB + koff[s]);
    u32x2 vlo[2][NT], vhi[2][NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      vlo[0][T] = vread(0, T);
      vhi[0][T] = vread(1, T);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sc[CT][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        sc[c][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) sc[c][u] = mfma_16x16x32<BF>(kf[u][s], qv[c][s], sc[c][u]);
      }
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      vlo[1][T] = vread(2, T);
      vhi[1][T] = vread(3, T);
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x2 pop[CT][4];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      float x[4][4];
      float mx;
      if constexpr (MASKED) {
        mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[u][e] = (tok0 + 16 * u + 4 * grp + e < lim[c]) ? sc[c][u][e] * c2 : -INFINITY;
            mx = fmaxf(mx, x[u][e]);
          }
      } else {
        // max of c2 * s over the stage = c2 * (max s, or min s for a negative scale)
        float r = sc[c][0][0];
        if (c2 >= 0.f) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) r = fmaxf(r, sc[c][u][e]);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) r = fminf(r, sc[c][u][e]);
        }
        mx = r * c2;
      }
      mx = max_rows32(max_rows16(mx));
      if (__ballot(mx > m[c]) != 0) {
        const float mn = fmaxf(m[c], mx);
        const float alpha = m[c] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[c] - mn);
        m[c] = mn;
        accL[c] *= alpha;
#pragma unroll
        for (int T = 0; T < NT; ++T) acc[c][T] *= alpha;
      }
      const float mb = m[c] == -INFINITY ? 0.f : m[c];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pr[e] = __builtin_amdgcn_exp2f(MASKED ? x[u][e] - mb : __builtin_fmaf(sc[c][u][e], c2, -mb));
        pop[c][u] = u32x2{pack2_16<BF>(pr[0], pr[1]), pack2_16<BF>(pr[2], pr[3])};
      }
    }
    u32x2 vm[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      vm[u] = u32x2{0xffffffffu, 0xffffffffu};
      if constexpr (MASKED) {
        const int tb = tok0 + 16 * u + 4 * grp;
        if (wlim - (tok0 + 16 * u) < 16) {
          vm[u].x = ((tb + 0 < wlim) ? 0x0000ffffu : 0u) | ((tb + 1 < wlim) ? 0xffff0000u : 0u);
          vm[u].y = ((tb + 2 < wlim) ? 0x0000ffffu : 0u) | ((tb + 3 < wlim) ? 0xffff0000u : 0u);
        }
      }
    }
    // P^T row sums (the softmax denominators) come from the matrix cores: an A operand of
    // bf16/f16 ones against the same P^T tile adds sum_t p to every row of accL, so the running
    // sum is rescaled with the output and needs no cross-lane reduction.
    const unsigned one2 = BF ? 0x3f803f80u : 0x3c003c00u;
    const u32x4 ones = {one2, one2, one2, one2};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 pb[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        pb[c] = u32x4{pop[c][2 * h].x, pop[c][2 * h].y, pop[c][2 * h + 1].x, pop[c][2 * h + 1].y};
        accL[c] = mfma_16x16x32<BF>(ones, pb[c], accL[c]);
      }
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        const u32x2 lo = vlo[h][T];
        const u32x2 hi = vhi[h][T];
        u32x4 va;
        if constexpr (MASKED)
          va = u32x4{lo.x & vm[2 * h].x, lo.y & vm[2 * h].y, hi.x & vm[2 * h + 1].x, hi.y & vm[2 * h + 1].y};
        else
          va = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[c][T] = mfma_16x16x32<BF>(va, pb[c], acc[c][T]);
      }
    }
  }

  // Column tile c: normalised output (or partial) row of this lane's column, d = 16 T + 4 grp ..
  __device__ __forceinline__ float denom(int c) const { return accL[c][0]; }
};

// Runs the stages [t_lo, tend) of one token range for every wave of the workgroup: prefetch
// stage s + 1 into registers, compute stage s from LDS buffer s & 1, store stage s + 1 into the
// other buffer, one barrier.  Every wave passes the same barriers (the same number of stages);
// the stages every column of a wave sees whole come first and take the unmasked compute.
// Expects stage 0 in LDS buffer 0 and the ids of stage 1 loaded (stage_prologue).
template <int D, int KV, bool BF, int NW, int CT>
__device__ __forceinline__ void run_stages(Stages<D, KV, BF, NW>& stg, ColTiles<D, BF, CT>& cols, const StageSrc& src,
                                           char* smem, int tid, int t_lo, int tend, bool active, float c2) {
  using SG = StageGeom<D, KV>;
  const int nst = (tend - t_lo + kStage - 1) / kStage;
  auto stage = [&](int s, char* cur, char* nxt, auto masked_tag) {
    const bool more = s + 1 < nst;                              // uniform over the workgroup
    if (more) {
      stg.load(src, tid, t_lo + (s + 1) * kStage, tend);
      stg.load_ids(src, tid, t_lo + (s + 2) * kStage, tend);
    }
    if (active) cols.template compute<decltype(masked_tag)::value>(cur, t_lo + s * kStage, c2);
    if (more) stg.store(nxt, tid);
    __syncthreads();
  };
  int nfast = active ? (cols.wmin - t_lo) / kStage : 0;
  nfast = nfast < 0 ? 0 : (nfast > nst ? nst : nfast);
  char* const buf0 = smem;
  char* const buf1 = smem + SG::STAGE;
  int s = 0;
  // unrolled by two so the LDS buffer offsets are immediates
  for (; s + 2 <= nfast; s += 2) {
    stage(s, buf0, buf1, std::false_type{});
    stage(s + 1, buf1, buf0, std::false_type{});
  }
  if (s < nfast) {
    stage(s, buf0, buf1, std::false_type{});
    ++s;
  }
  for (; s < nst; ++s) stage(s, (s & 1) ? buf1 : buf0, (s & 1) ? buf0 : buf1, std::true_type{});
}

// Stage 0 of [t_lo, tend) into LDS buffer 0, the ids of stage 1 loaded, one barrier.
template <int D, int KV, bool BF, int NW>
__device__ __forceinline__ void stage_prologue(Stages<D, KV, BF, NW>& stg, const StageSrc& src, char* smem, int tid,
                                               int t_lo, int tend) {
  stg.load_ids(src, tid, t_lo, tend);
  stg.load(src, tid, t_lo, tend);
  stg.load_ids(src, tid, t_lo + kStage, tend);
  stg.store(smem, tid);
  __syncthreads();
}

// ---- the shared-prefix pass
// Configuration: eight waves of one 16-column tile (128 query columns per workgroup), two waves
// per SIMD; four waves of two tiles (one wave per SIMD, half the LDS reads per column) measured
// slower.
constexpr int kPrefixWaves = 8;
constexpr int kPrefixCT = 1;
constexpr int kPrefixCols = 16 * kPrefixCT * kPrefixWaves;   // query columns per workgroup

struct PrefixParams {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;      // the first entries of row 0 are the prefix's blocks
  const int32_t* lens;
  float* tmp_out;
  float* max_logits;
  float* exp_sums;
  int B, Hq, Hkv, G, num_blocks, cap, max_blocks;
  int bs_shift;           // log2(block_size)
  int prefix_len;         // tokens of the shared prefix, a multiple of 16
  int chunk;              // tokens per prefix partition, a multiple of 16
  int parts;              // prefix partitions
  int hp8;                // Hkv * parts rounded up to a multiple of 8 (the grid's stride)
  int Pslots;
  float c2, v_scale;
};

// One workgroup per (KV head, prefix partition, block of query columns); column c of the batch
// is (sequence c / G, head g * G + c % G) and sees the first min(n, prefix_len) tokens.  The
// result is one (m, l, o) partial per (row, head, prefix partition), merged with the suffix
// partials by the reduce.
// One tile per wave fits two waves per SIMD; two tiles per wave take the whole register file.
template <int D, int KV, bool BF, int NW, int CT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(CT == 1 ? 2 : 1)))
void pa_prefix_kernel(PrefixParams a) {
  constexpr int COLS = 16 * CT * NW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wl = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroup w = hc + hp8 * qb: (KV head, partition) hc, query block qb.  Workgroups are dealt
  // to the 8 XCDs round-robin by w, so all query blocks of one (head, partition) land on the
  // same XCD and read its slice of the prefix through one L2.
  const int hc = blockIdx.x % a.hp8;
  const int qb = blockIdx.x / a.hp8;
  if (hc >= a.Hkv * a.parts) return;                          // padding of the stride
  const int g = hc % a.Hkv;                                   // KV head
  const int part = hc / a.Hkv;
  const int c0 = part * a.chunk;                              // the partition: tokens [c0, c1)
  const int c1 = min(c0 + a.chunk, a.prefix_len);
  StageSrc src;
  src.rowstride = a.Hkv * StageGeom<D, KV>::ROWB;
  src.kc = (const char*)a.kc + (size_t)g * StageGeom<D, KV>::ROWB;
  src.vc = (const char*)a.vc + (size_t)g * StageGeom<D, KV>::ROWB;
  src.row = a.bt;
  src.blockbytes = (size_t)src.rowstride << a.bs_shift;
  src.bs_shift = a.bs_shift;
  src.lastcol = a.max_blocks - 1;
  src.nbm1 = (unsigned)(a.num_blocks - 1);

  Stages<D, KV, BF, NW> stg;
  stg.load_ids(src, tid, c0, c1);
  stg.load(src, tid, c0, c1);
  stg.load_ids(src, tid, c0 + kStage, c1);

  // ---- this wave's columns (V rows at or past every column's limit are masked: such slots of
  // shared blocks may hold stale bytes)
  const int BG = a.B * a.G;
  const int cb = qb * COLS + wl * 16 * CT;
  const bool active = cb < BG;                                // wave-uniform
  ColTiles<D, BF, CT> cols;
  cols.init(lane);
  cols.reset();
  int bcol[CT], hcol[CT];
  bool cvalid[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int col = cb + 16 * c + (lane & 15);
    cvalid[c] = col < BG;
    const int cc = cvalid[c] ? col : BG - 1;
    bcol[c] = cc / a.G;
    hcol[c] = g * a.G + (cc - bcol[c] * a.G);
    cols.lim[c] = cvalid[c] ? min(min(clamp_len(a.lens[bcol[c]], a.cap), a.prefix_len), c1) : 0;
    cols.load_q(c, (const char*)a.q + ((size_t)bcol[c] * a.Hq + hcol[c]) * D * 2);
  }
  cols.limits_done();
  stg.store(smem, tid);
  // q must be resident before the loop: loads retire in order, so a q load still counted as
  // outstanding inside the loop would make the first MFMA wait for the next stage's prefetch.
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int s = 0; s < StageGeom<D, KV>::NS; ++s) asm volatile("" : : "v"(cols.qv[c][s]));
  __syncthreads();
  run_stages(stg, cols, src, smem, tid, c0, c1, active, a.c2);

  if (!active) return;
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const float l = cols.denom(c);
    const float inv = l > 0.f ? a.v_scale / l : 0.f;
    if (cvalid[c]) {
      const size_t prow = ((size_t)bcol[c] * a.Hq + hcol[c]) * a.Pslots + part;
      float* orow = a.tmp_out + prow * D;
#pragma unroll
      for (int T = 0; T < StageGeom<D, KV>::NT; ++T) *(f32x4*)(orow + 16 * T + 4 * cols.grp) = cols.acc[c][T] * inv;
      if (cols.grp == 0) {
        a.max_logits[prow] = cols.m[c] * kLn2;
        a.exp_sums[prow] = l;
      }
    }
  }
}

// ---- multi-query attention with many new tokens per sequence
// A workgroup of NW waves of CT 16-column tiles serves one KV head, one block of NW * CT * 16
// (head, new token) columns and the token ranges of its schedule.

// grid.y = g * col_blocks + column block.  Column c of a sequence's block is (query head
// g * G + c / L, new token i = c % L); token i sits at position n - L + i and sees the first
// n - (L - 1 - i) tokens.  Modes: one workgroup per sequence (final rows), per fixed partition
// or per range of the balanced split (partials for paged_attn_reduce over L * Hq rows).
template <int D, int KV, bool BF, int MODE, int NW, int CT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(CT == 1 ? 2 : 1)))
void pa_mq_tiled_kernel(DecodeParams a, int col_blocks) {
  constexpr int COLS = 16 * CT * NW;
  using SG = StageGeom<D, KV>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wl = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.y / col_blocks;
  const int cbk = blockIdx.y - g * col_blocks;
  const int GL = a.G * a.L;
  const int cb = cbk * COLS + wl * 16 * CT;                   // the wave's first column
  const bool active = cb < GL;                                // wave-uniform
  const int cap = a.cap;

  SegSource segs;
  segs.mode = MODE;
  segs.w = 0;
  Seg cur;
  if constexpr (MODE == MODE_SINGLE) {
    cur.b = blockIdx.x;
    cur.n = clamp_len(__builtin_amdgcn_readfirstlane(a.lens[cur.b]), cap);
    cur.tlo = 0;
    cur.thi = (cur.n + 15) >> 4;
    cur.slot = -1;
    cur.valid = true;
  } else if constexpr (MODE == MODE_FIXED) {
    cur.b = blockIdx.z;
    cur.n = clamp_len(__builtin_amdgcn_readfirstlane(a.lens[cur.b]), cap);
    cur.slot = blockIdx.x;
    cur.tlo = (cur.slot * a.PS) >> 4;
    cur.thi = (min((cur.slot + 1) * a.PS, cur.n) + 15) >> 4;
    cur.valid = cur.thi > cur.tlo;
    if (!cur.valid) return;
  } else {
    if (!balanced_start(segs, cur, a.lens, a.B, cap, 0, a.W, blockIdx.x, lane)) return;
  }

  StageSrc src;
  src.rowstride = a.Hkv * SG::ROWB;
  src.kc = (const char*)a.kc + (size_t)g * SG::ROWB;
  src.vc = (const char*)a.vc + (size_t)g * SG::ROWB;
  src.blockbytes = (size_t)src.rowstride * a.BS;
  src.bs_shift = a.tile_shift + 4;
  src.lastcol = a.max_blocks - 1;
  src.nbm1 = (unsigned)(a.num_blocks - 1);

  Stages<D, KV, BF, NW> stg;
  ColTiles<D, BF, CT> cols;
  cols.init(lane);
  int hcol[CT], icol[CT];
  bool cvalid[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int col = cb + 16 * c + (lane & 15);
    cvalid[c] = col < GL;
    const int cc = cvalid[c] ? col : 0;
    hcol[c] = g * a.G + cc / a.L;
    icol[c] = cc % a.L;
  }

  for (;;) {
    // ---- one segment: tokens [t_lo, tend) of sequence cur.b
    const int t_lo = cur.tlo << 4;
    const int tend = min(cur.thi << 4, cur.n);
    src.row = a.bt + (size_t)cur.b * a.max_blocks;
    stg.load_ids(src, tid, t_lo, tend);
    stg.load(src, tid, t_lo, tend);
    stg.load_ids(src, tid, t_lo + kStage, tend);
    cols.reset();
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      cols.lim[c] = cvalid[c] ? min(cur.n - (a.L - 1 - icol[c]), tend) : 0;
      cols.load_q(c, (const char*)a.q + (((size_t)cur.b * a.L + icol[c]) * a.Hq + hcol[c]) * D * 2);
    }
    cols.limits_done();
    stg.store(smem, tid);
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int s = 0; s < SG::NS; ++s) asm volatile("" : : "v"(cols.qv[c][s]));
    __syncthreads();
    run_stages(stg, cols, src, smem, tid, t_lo, tend, active, a.c2);

    // ---- the segment's rows: final output (single pass) or a partial
    if (active) {
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        if (!cvalid[c]) continue;
        const float l = cols.denom(c);
        const float inv = l > 0.f ? a.v_scale / l : 0.f;
        const size_t row = ((size_t)cur.b * a.L + icol[c]) * a.Hq + hcol[c];
        if constexpr (MODE == MODE_SINGLE) {
          unsigned short* orow = (unsigned short*)a.out + row * D;
#pragma unroll
          for (int T = 0; T < SG::NT; ++T) {
            u32x2 wv;
            wv.x = pack2_16<BF>(cols.acc[c][T][0] * inv, cols.acc[c][T][1] * inv);
            wv.y = pack2_16<BF>(cols.acc[c][T][2] * inv, cols.acc[c][T][3] * inv);
            *(u32x2*)(orow + 16 * T + 4 * cols.grp) = wv;
          }
        } else if (cur.slot >= 0 && cur.slot < a.Pslots) {
          const size_t prow = row * a.Pslots + cur.slot;
          float* orow = a.tmp_out + prow * D;
#pragma unroll
          for (int T = 0; T < SG::NT; ++T) *(f32x4*)(orow + 16 * T + 4 * cols.grp) = cols.acc[c][T] * inv;
          if (cols.grp == 0) {
            a.max_logits[prow] = cols.m[c] * kLn2;
            a.exp_sums[prow] = l;
          }
        }
      }
    }
    if constexpr (MODE != MODE_BALANCED) break;
    cur = segs.next(cur, lane);
    if (!cur.valid) break;
  }
}

// ------------------------------------------------------------------ split-K reduce

// One wave per output row (sequence b, query head h); four rows per workgroup.  PS > 0:
// partials of fixed partitions, P = ceil(n / PS).  PS < 0: balanced split over -PS
// workgroups; P = number of ranges the sequence's tiles (past its first t0) fall in,
// recomputed from the lengths exactly as the decode did.  slot0 leading slots (a shared
// prefix's partials) come before those P.  compact: the balanced split's compact layout (partial
// b + w of row h sits at [b + w][h]; see DecodeParams).  No LDS and no barrier: 16-lane row r of
// the wave folds the partials p = r, r+4, ... into a running (max, weight sum, weighted o) over
// its D/16 output elements per lane, and the four rows are combined with permlane swaps.
template <int D, bool BF>
__global__ __launch_bounds__(256) void pa_reduce_kernel(void* out, const float* tmp_out,
                                                       const float* max_logits,
                                                       const float* exp_sums,
                                                       const int32_t* lens, int B, int Hq,
                                                       int Pslots, int PS, int cap, int t0,
                                                       int slot0, int compact) {
  constexpr int DPL = D / 16;                 // output elements per lane (8 or 4)
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, l16 = lane & 15;
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // b * Hq + h
  if (row >= B * Hq) return;
  const int b = row / Hq;
  const int n = clamp_len(__builtin_amdgcn_readfirstlane(lens[b]), cap);
  int P, first_range = 0;
  if (PS > 0) {
    P = (n + PS - 1) / PS;
  } else {
    int total = 0, before = 0;               // split units of the whole batch, of sequences < b
    for (int i0 = 0; i0 < B; i0 += 64) {
      const int i = i0 + lane;
      const int u = i < B ? units_after(clamp_len(lens[i], cap), t0) : 0;
      total += u;
      before += i < b ? u : 0;
    }
    total = __builtin_amdgcn_readlane(wave_incl_scan(total), 63);
    before = __builtin_amdgcn_readlane(wave_incl_scan(before), 63);
    const int nt = tiles_after(n, t0);
    if (nt == 0) {
      P = 0;
    } else {
      const Split split(total, -PS);
      const int first = before + 1;          // the unit of b's first tile
      first_range = split.owner(first);
      P = split.owner(first + nt - 1) - first_range + 1;
    }
  }
  if (!compact) P = min(slot0 + P, Pslots);
  unsigned short* orow = (unsigned short*)out + (size_t)row * D + l16 * DPL;
  if (P == 0) {
    if (grp == 0) {
      if constexpr (DPL == 8)
        *(u32x4*)orow = u32x4{0u, 0u, 0u, 0u};
      else
        *(u32x2*)orow = u32x2{0u, 0u};
    }
    return;
  }
  // partial p of this row: index base + p * pstride of max_logits / exp_sums (times D for tmp_out)
  const size_t base = compact ? (size_t)(b + first_range) * Hq + (row - b * Hq) : (size_t)row * Pslots;
  const size_t pstride = compact ? (size_t)Hq : 1;
  const float* ml = max_logits + base;
  const float* es = exp_sums + base;
  const float* to = tmp_out + base * D + l16 * DPL;

  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  float mrun = -INFINITY, wrun = 0.f;
#pragma unroll 4
  for (int p = grp; p < P; p += 4) {
    const float mp = ml[p * pstride] * kLog2e;
    const float lp = es[p * pstride];
    float o[DPL];
#pragma unroll
    for (int i = 0; i < DPL; i += 4) {
      const f32x4 v = *(const f32x4*)(to + p * pstride * D + i);
      o[i] = v[0];
      o[i + 1] = v[1];
      o[i + 2] = v[2];
      o[i + 3] = v[3];
    }
    // a partial that saw no token (causal multi-query) has m = -inf and l = 0
    const float mn = fmaxf(mrun, mp);
    const float so = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mrun - mn);
    const float sn = mp == -INFINITY ? 0.f : lp * __builtin_amdgcn_exp2f(mp - mn);
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = acc[i] * so + o[i] * sn;
    wrun = wrun * so + sn;
    mrun = mn;
  }
  // combine the four rows: rescale each to the common maximum (a row without partials has
  // mrun = -inf and weight 0), then sum across rows
  const float M = max_rows32(max_rows16(mrun));
  const float sg = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - M);
  const float wsum = sum_rows32(sum_rows16(wrun * sg));
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = sum_rows32(sum_rows16(acc[i] * sg));
  if (grp == 0) {
    unsigned w[DPL / 2];
#pragma unroll
    for (int i = 0; i < DPL / 2; ++i)
      w[i] = pack2(f32_to_16<BF>(acc[2 * i] * inv), f32_to_16<BF>(acc[2 * i + 1] * inv));
    if constexpr (DPL == 8)
      *(u32x4*)orow = u32x4{w[0], w[1], w[2], w[3]};
    else
      *(u32x2*)orow = u32x2{w[0], w[1]};
  }
}

// Merge for launches with many output rows and few partials per row (multi-query: L * Hq rows
// per sequence, a narrow balanced split): each 16-lane group of a wave folds all partials of
// its own row, so a wave serves four rows instead of one.  Needs rows_per_seq >= 4, so the four
// rows of a wave belong to at most two consecutive sequences.  Same partial layout and the same
// partial counts as pa_reduce_kernel (non-compact layout).
template <int D, bool BF>
__global__ __launch_bounds__(256) void pa_reduce_rows_kernel(void* out, const float* tmp_out,
                                                            const float* max_logits, const float* exp_sums,
                                                            const int32_t* lens, int B, int Hq, int Pslots,
                                                            int PS, int cap, int t0, int slot0) {
  constexpr int DPL = D / 16;                 // output elements per lane (8 or 4)
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, l16 = lane & 15;
  const int r0 = (blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * 4;
  if (r0 >= B * Hq) return;
  const int row = r0 + grp;                   // this group's row (b * Hq + h)
  const bool live = row < B * Hq;
  const int b_lo = r0 / Hq;                   // the wave's first sequence
  const int b = live ? row / Hq : b_lo;       // b_lo or b_lo + 1
  const int n = clamp_len(lens[b], cap);
  int P, first_range = 0;
  if (PS > 0) {
    P = (n + PS - 1) / PS;
  } else {
    int total = 0, before = 0;               // split units of the whole batch, of sequences < b_lo
    for (int i0 = 0; i0 < B; i0 += 64) {
      const int i = i0 + lane;
      const int u = i < B ? units_after(clamp_len(lens[i], cap), t0) : 0;
      total += u;
      before += i < b_lo ? u : 0;
    }
    total = __builtin_amdgcn_readlane(wave_incl_scan(total), 63);
    before = __builtin_amdgcn_readlane(wave_incl_scan(before), 63);
    if (b > b_lo) before += units_after(clamp_len(__builtin_amdgcn_readfirstlane(lens[b_lo]), cap), t0);
    const int nt = tiles_after(n, t0);
    if (nt == 0) {
      P = 0;
    } else {
      const Split split(total, -PS);
      const int first = before + 1;          // the unit of b's first tile
      first_range = split.owner(first);
      P = split.owner(first + nt - 1) - first_range + 1;
    }
  }
  P = live ? min(slot0 + P, Pslots) : 0;
  const float* ml = max_logits + (size_t)row * Pslots;
  const float* es = exp_sums + (size_t)row * Pslots;
  const float* to = tmp_out + (size_t)row * Pslots * D + l16 * DPL;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  float mrun = -INFINITY, wrun = 0.f;
#pragma unroll 2
  for (int p = 0; p < P; ++p) {
    const float mp = ml[p] * kLog2e;
    const float lp = es[p];
    float o[DPL];
#pragma unroll
    for (int i = 0; i < DPL; i += 4) {
      const f32x4 v = *(const f32x4*)(to + (size_t)p * D + i);
      o[i] = v[0];
      o[i + 1] = v[1];
      o[i + 2] = v[2];
      o[i + 3] = v[3];
    }
    // a partial that saw no token (causal multi-query) has m = -inf and l = 0
    const float mn = fmaxf(mrun, mp);
    const float so = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mrun - mn);
    const float sn = mp == -INFINITY ? 0.f : lp * __builtin_amdgcn_exp2f(mp - mn);
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = acc[i] * so + o[i] * sn;
    wrun = wrun * so + sn;
    mrun = mn;
  }
  if (!live) return;
  const float inv = wrun > 0.f ? 1.0f / wrun : 0.f;
  unsigned w[DPL / 2];
#pragma unroll
  for (int i = 0; i < DPL / 2; ++i) w[i] = pack2(f32_to_16<BF>(acc[2 * i] * inv), f32_to_16<BF>(acc[2 * i + 1] * inv));
  unsigned short* orow = (unsigned short*)out + (size_t)row * D + l16 * DPL;
  if constexpr (DPL == 8)
    *(u32x4*)orow = u32x4{w[0], w[1], w[2], w[3]};
  else
    *(u32x2*)orow = u32x2{w[0], w[1]};
}

// ------------------------------------------------------------------ KV write scatter

// Row i of key/value (row_elems elements each) into slot s of the caches; the calling
// workgroup's threads each move 8 elements (16 source bytes) per step.
template <bool SRC_BF, bool TO_FP8>
__device__ __forceinline__ void write_row(const void* key, const void* value, void* key_cache, void* value_cache,
                                          long long i, long long s, int row_elems, float k_scale,
                                          float v_scale) {
  const int chunks = row_elems >> 3;
  for (int c = threadIdx.x; c < 2 * chunks; c += 256) {
    const bool isv = c >= chunks;
    const int cc = isv ? c - chunks : c;
    const u32x4 x = *(const u32x4*)((const char*)(isv ? value : key) +
                                    ((size_t)i * row_elems + (size_t)cc * 8) * 2);
    char* cache = (char*)(isv ? value_cache : key_cache);
    if constexpr (!TO_FP8) {
      *(u32x4*)(cache + ((size_t)s * row_elems + (size_t)cc * 8) * 2) = x;
    } else {
      const float sc = isv ? v_scale : k_scale;
      unsigned codes[8];
      const unsigned w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const unsigned short hbits = (unsigned short)(w[e >> 1] >> (16 * (e & 1)));
        const float v = from16<SRC_BF>(hbits);
        codes[e] = e4m3fn_code(v / sc);                 // IEEE fp32 division
      }
      u32x2 o;
      o.x = codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24);
      o.y = codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24);
      *(u32x2*)(cache + (size_t)s * row_elems + (size_t)cc * 8) = o;
    }
  }
}

// One workgroup per new token.
template <bool SRC_BF, bool TO_FP8>
__global__ __launch_bounds__(256) void kv_write_kernel(const void* key, const void* value,
                                                      void* key_cache, void* value_cache,
                                                      const int64_t* slots, long long nslots,
                                                      int row_elems, float k_scale,
                                                      float v_scale) {
  const int i = blockIdx.x;
  const long long s = slots[i];
  if (s < 0 || s >= nslots) return;
  write_row<SRC_BF, TO_FP8>(key, value, key_cache, value_cache, i, s, row_elems, k_scale, v_scale);
}

// One workgroup per sequence: its new row goes to position n - 1, the slot read from the
// block table (ids clamped into the pool); sequences with n = 0 have no new token.
__global__ __launch_bounds__(256) void kv_append_kernel(const void* key, const void* value, void* key_cache,
                                                       void* value_cache, const int32_t* bt,
                                                       const int32_t* lens, int max_blocks, int cap,
                                                       int bs_shift, int num_blocks, int row_elems) {
  const int b = blockIdx.x;
  const int n = clamp_len(lens[b], cap);
  if (n == 0) return;
  const int t = n - 1;
  const int col = min(t >> bs_shift, max_blocks - 1);   // a length past the table: its last entry
  const unsigned id = min((unsigned)bt[(size_t)b * max_blocks + col], (unsigned)(num_blocks - 1));
  const long long s = ((long long)id << bs_shift) + (t & ((1 << bs_shift) - 1));
  write_row<true, false>(key, value, key_cache, value_cache, b, s, row_elems, 1.f, 1.f);
}

// ------------------------------------------------------------------ host helpers

// Measurement hook (pkv_time_next_call): the caller's events, bound to the kernels of the next
// attention call on this thread -- the start event to the call's first kernel, the stop event to
// its last -- so that the elapsed time between them is the kernels' own execution time.
struct CallTimer {
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local CallTimer t_armed;   // set by pkv_time_next_call, taken by the next attention call
thread_local CallTimer t_call;    // the running call's events
thread_local bool t_first = true; // the running call has not launched a kernel yet

// Scope of one attention call: takes the armed events (a call that fails its checks drops them).
struct TimedCall {
  TimedCall() {
    t_call = std::exchange(t_armed, CallTimer{});
    t_first = true;
  }
  ~TimedCall() { t_call = CallTimer{}; }
};

// Every kernel of an attention call is launched here.  `last` marks the call's final kernel.
// With events bound, hipExtLaunchKernel records them at the kernel's start and end; otherwise a
// plain launch.
template <typename F, typename... Args>
void launch(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st, bool last, Args... args) {
  const hipEvent_t e0 = t_first ? t_call.start : nullptr;
  const hipEvent_t e1 = last ? t_call.stop : nullptr;
  t_first = false;
  if (e0 || e1)
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)lds, st, e0, e1, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
}

// New query tokens per sequence accepted by paged_attn_multi_query.
constexpr int kMaxQueryLen = 4096;

// Partial slots per (sequence, head): fixed partitions need ceil(max_len / PS); a balanced
// split gives every workgroup >= kMinChunkTiles units, and a sequence's tiles are consecutive
// units, so a sequence meets at most ceil(tiles / kMinChunkTiles) + 1 ranges.
int slots_of(int max_context_len, int partition_size) {
  if (partition_size > 0) return (max_context_len + partition_size - 1) / partition_size;
  if (partition_size < 0) {
    const int tiles = (max_context_len + 15) / 16;
    return tiles == 0 ? 0 : (tiles + kMinChunkTiles - 1) / kMinChunkTiles + 1;
  }
  return 0;
}

int waves_per_group(int Hkv) { return Hkv < kMaxWaves ? Hkv : kMaxWaves; }
int head_groups(int Hkv) { return (Hkv + kMaxWaves - 1) / kMaxWaves; }

template <int D, int KV, bool BF, int POLICY, int CT>
void launch_decode_policy(const DecodeParams& p, bool last, hipStream_t st) {
  const int HG = head_groups(p.Hkv);
  const int nw = waves_per_group(p.Hkv);
  const size_t lds = (size_t)nw * Tile<D, KV, CT>::LDS_BYTES;
  if (p.mode == MODE_SINGLE)
    launch(pa_decode_kernel<D, KV, BF, MODE_SINGLE, POLICY, false, CT>, dim3(p.B, HG), dim3(64 * nw), lds, st, last,
           p);
  else if (p.mode == MODE_FIXED)
    launch(pa_decode_kernel<D, KV, BF, MODE_FIXED, POLICY, false, CT>, dim3(p.Pslots, HG, p.B), dim3(64 * nw), lds, st,
           last, p);
  else
    launch(pa_decode_kernel<D, KV, BF, MODE_BALANCED, POLICY, false, CT>, dim3(p.W, HG), dim3(64 * nw), lds, st, last,
           p);
}

// Columns (head, new token) per KV group that the decode kernel carries (two MFMA tiles per wave).
constexpr int kDecodeMaxCols = 32;

// Multi-query with more (head, new token) columns than a decode wave carries: the tiled kernel,
// one workgroup per (work item, KV head, block of kMqCols columns).  Eight waves of one
// 16-column tile, two waves per SIMD: measured faster than four waves (one per SIMD) of two
// tiles each, and than four-wave workgroups of one tile, at every q_len tried.
constexpr int kMqWaves = 8, kMqCT = 1;
constexpr int kMqCols = 16 * kMqWaves * kMqCT;
int mq_col_blocks(int G, int L) { return (G * L + kMqCols - 1) / kMqCols; }

template <int D, int KV, bool BF, int NW, int CT>
void launch_mq_tiled_cfg(const DecodeParams& p, bool last, hipStream_t st) {
  const int CB = mq_col_blocks(p.G, p.L);
  const unsigned gy = (unsigned)(p.Hkv * CB);
  const size_t lds = (size_t)StageGeom<D, KV>::LDS_BYTES;
  const dim3 block(64 * NW);
  if (p.mode == MODE_SINGLE)
    launch(pa_mq_tiled_kernel<D, KV, BF, MODE_SINGLE, NW, CT>, dim3(p.B, gy), block, lds, st, last, p, CB);
  else if (p.mode == MODE_FIXED)
    launch(pa_mq_tiled_kernel<D, KV, BF, MODE_FIXED, NW, CT>, dim3(p.Pslots, gy, p.B), block, lds, st, last, p, CB);
  else
    launch(pa_mq_tiled_kernel<D, KV, BF, MODE_BALANCED, NW, CT>, dim3(p.W, gy), block, lds, st, last, p, CB);
}

// Tiled multi-query workgroups resident per compute unit (balanced schedule) for this shape.
template <int D, int KV, bool BF>
int mq_occupancy() {
  int nb = 0;
  const size_t lds = (size_t)StageGeom<D, KV>::LDS_BYTES;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &nb, (const void*)pa_mq_tiled_kernel<D, KV, BF, MODE_BALANCED, kMqWaves, kMqCT>, 64 * kMqWaves, lds);
  return e == hipSuccess && nb > 0 ? nb : 1;
}

template <int D, int KV, bool BF>
void launch_mq_tiled(const DecodeParams& p, bool last, hipStream_t st) {
  launch_mq_tiled_cfg<D, KV, BF, kMqWaves, kMqCT>(p, last, st);
}

// The balanced decode with the step's new rows appended in the same launch (16-bit caches).
template <int D, int KV, bool BF>
void launch_decode_append(const DecodeParams& p, bool shared_blocks, hipStream_t st) {
  const int HG = head_groups(p.Hkv);
  const int nw = waves_per_group(p.Hkv);
  const size_t lds = (size_t)nw * Tile<D, KV>::LDS_BYTES;
  if (shared_blocks)
    launch(pa_decode_kernel<D, KV, BF, MODE_BALANCED, kCachedPolicy, true>, dim3(p.W, HG), dim3(64 * nw), lds, st,
           true, p);
  else
    launch(pa_decode_kernel<D, KV, BF, MODE_BALANCED, kStreamPolicy, true>, dim3(p.W, HG), dim3(64 * nw), lds, st,
           true, p);
}

// Up to 16 (head, new token) columns per KV group: one MFMA tile per wave; up to 32: two.
template <int D, int KV, bool BF>
void launch_decode(const DecodeParams& p, bool shared_blocks, bool last, hipStream_t st) {
  const bool two = p.G * p.L > 16;
  if (shared_blocks) {
    if (two) launch_decode_policy<D, KV, BF, kCachedPolicy, 2>(p, last, st);
    else launch_decode_policy<D, KV, BF, kCachedPolicy, 1>(p, last, st);
  } else {
    if (two) launch_decode_policy<D, KV, BF, kStreamPolicy, 2>(p, last, st);
    else launch_decode_policy<D, KV, BF, kStreamPolicy, 1>(p, last, st);
  }
}

template <int D, int KV, bool BF>
void launch_prefix(const PrefixParams& p, hipStream_t st) {
  const long long qblocks = ((long long)p.B * p.G + kPrefixCols - 1) / kPrefixCols;
  const dim3 grid((unsigned)(qblocks * p.hp8));
  const size_t lds = (size_t)StageGeom<D, KV>::LDS_BYTES;
  launch(pa_prefix_kernel<D, KV, BF, kPrefixWaves, kPrefixCT>, grid, dim3(64 * kPrefixWaves), lds, st, false, p);
}

// Output rows from which a merge serves four rows per wave (pa_reduce_rows_kernel).
constexpr long long kReduceRowsPerGroupMin = 16384;

void launch_reduce(void* out, const float* tmp_out, const float* max_logits, const float* exp_sums,
                   const int32_t* lens, int B, int rows_per_seq, int D, int Pslots, int PS, int cap,
                   int t0, int slot0, bool bf, hipStream_t st, int compact = 0) {
  const long long rows = (long long)B * rows_per_seq;
  const int Pm = Pslots > 0 ? Pslots : 1;
  if (!compact && rows_per_seq >= 4 && rows >= kReduceRowsPerGroupMin) {
    const dim3 grid((unsigned)((rows + 15) / 16)), block(256);
    auto k = D == 128 ? (bf ? pa_reduce_rows_kernel<128, true> : pa_reduce_rows_kernel<128, false>)
                      : (bf ? pa_reduce_rows_kernel<64, true> : pa_reduce_rows_kernel<64, false>);
    launch(k, grid, block, 0, st, true, out, tmp_out, max_logits, exp_sums, lens, B, rows_per_seq, Pm, PS, cap, t0,
           slot0);
    return;
  }
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  auto k = D == 128 ? (bf ? pa_reduce_kernel<128, true> : pa_reduce_kernel<128, false>)
                    : (bf ? pa_reduce_kernel<64, true> : pa_reduce_kernel<64, false>);
  launch(k, grid, block, 0, st, true, out, tmp_out, max_logits, exp_sums, lens, B, rows_per_seq, Pm, PS, cap, t0,
         slot0, compact);
}

// Partial slots of a shared-prefix decode: the prefix partitions first, then the balanced
// split of the suffix (the tokens past the prefix).
int prefix_parts(int prefix_len, int prefix_partition_size) {
  return prefix_len > 0 ? (prefix_len + prefix_partition_size - 1) / prefix_partition_size : 0;
}
int shared_prefix_slots(int max_context_len, int prefix_len, int prefix_partition_size, int partition_size) {
  const int suffix = max_context_len > prefix_len ? max_context_len - prefix_len : 0;
  return prefix_parts(prefix_len, prefix_partition_size) + slots_of(suffix, partition_size);
}

template <int D, int KV, bool BF>
int occupancy_blocks(int Hkv) {
  int nb = 0;
  const int nw = waves_per_group(Hkv);
  const size_t lds = (size_t)nw * Tile<D, KV>::LDS_BYTES;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &nb, (const void*)pa_decode_kernel<D, KV, BF, MODE_BALANCED, kStreamPolicy>, 64 * nw, lds) != hipSuccess)
    return 0;
  return nb;
}

}  // namespace

// ------------------------------------------------------------------ fixed scratch (no allocation)

// Split-K partials of paged_attn_decode_noalloc: a fixed device array, one copy per GPU the
// library runs on, held until the process ends.  Host code never uses its name as an address
// (that is a host-side stand-in); the device address comes from hipGetSymbolAddress, once per
// device.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};

// Device address of the current device's `scratch`.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PKV_ERR_LAUNCH;
    scratch_dev[dev] = ptr;
  }
  *out = scratch_dev[dev];
  return PKV_OK;
}
}  // namespace

// ==================================================================== C ABI

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "a size is negative, inconsistent or unsupported";
    case PKV_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case PKV_ERR_ALIGN: return "a pointer is not aligned as required";
    case PKV_ERR_WORKSPACE: return "split-K workspace buffers missing";
    case PKV_ERR_LAUNCH: return "HIP kernel launch failed";
    case PKV_ERR_CHECK: return "checked mode found an invalid device-resident value";
    case PKV_ERR_STATE: return "sequence id already used, or the sequence is in the wrong state";
    case PKV_ERR_NOT_FOUND: return "unknown sequence id";
    case PKV_ERR_NO_SPACE: return "not enough free blocks";
    case PKV_ERR_HOST: return "host buffer is not pinned, mapped host memory of the required size";
    case PKV_ERR_SCRATCH: return "the call needs more scratch than the library's fixed device buffer holds";
    default: return "unknown status";
  }
}

int pkv_time_next_call(void* start_event, void* stop_event) {
  t_armed.start = (hipEvent_t)start_event;
  t_armed.stop = (hipEvent_t)stop_event;
  return PKV_OK;
}

int paged_attn_partial_slots(int max_context_len, int partition_size) {
  if (max_context_len <= 0) return 0;
  return slots_of(max_context_len, partition_size);
}

size_t paged_attn_workspace_bytes(int num_seqs, int num_heads, int head_dim, int max_context_len,
                                  int partition_size) {
  if (partition_size == 0 || num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0)
    return 0;
  const size_t P = (size_t)slots_of(max_context_len, partition_size);
  return (size_t)num_seqs * num_heads * P * ((size_t)head_dim + 2) * sizeof(float);
}

int paged_attn_balanced_split(int num_kv_heads, int head_dim, int q_dtype, int kv_dtype) {
  if (num_kv_heads <= 0 || num_kv_heads > 16 || (head_dim != 64 && head_dim != 128)) return 0;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  const bool bf = q_dtype == PKV_BF16, f8 = kv_dtype == PKV_FP8_E4M3;
  int nb;
  if (head_dim == 128)
    nb = f8 ? (bf ? occupancy_blocks<128, KFP8, true>(num_kv_heads) : occupancy_blocks<128, KFP8, false>(num_kv_heads))
            : (bf ? occupancy_blocks<128, KBF16, true>(num_kv_heads) : occupancy_blocks<128, KF16, false>(num_kv_heads));
  else
    nb = f8 ? (bf ? occupancy_blocks<64, KFP8, true>(num_kv_heads) : occupancy_blocks<64, KFP8, false>(num_kv_heads))
            : (bf ? occupancy_blocks<64, KBF16, true>(num_kv_heads) : occupancy_blocks<64, KF16, false>(num_kv_heads));
  if (nb <= 0) nb = 1;
  const int w = prop.multiProcessorCount * nb / head_groups(num_kv_heads);
  return -(w > 0 ? w : 1);
}

int paged_kv_write(const void* key, const void* value, void* key_cache, void* value_cache,
                   const int64_t* slot_mapping, int num_tokens, int num_blocks, int block_size,
                   int num_kv_heads, int head_dim, int src_dtype, int cache_dtype, float k_scale,
                   float v_scale, void* stream) {
  if (num_tokens < 0 || num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return PKV_ERR_SHAPE;
  if (src_dtype != PKV_F16 && src_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (cache_dtype != src_dtype && cache_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  const bool to_fp8 = cache_dtype == PKV_FP8_E4M3;
  if (head_dim % (to_fp8 ? 16 : 8) != 0) return PKV_ERR_SHAPE;
  if (to_fp8 && !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(slot_mapping, 8))
    return PKV_ERR_ALIGN;
  const long long nslots = (long long)num_blocks * block_size;
  const long long row = (long long)num_kv_heads * head_dim;
  if (row > (1 << 24)) return PKV_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (check_mode()) {
    std::vector<int64_t> sm;
    if (!copy_to_host(sm, slot_mapping, (size_t)num_tokens, st)) return PKV_ERR_LAUNCH;
    std::vector<char> seen((size_t)nslots, 0);
    for (int64_t s : sm) {
      if (s < 0) continue;
      if (s >= nslots || seen[(size_t)s]) return PKV_ERR_CHECK;
      seen[(size_t)s] = 1;
    }
  }
  dim3 grid(num_tokens), block(256);
  const bool bf = src_dtype == PKV_BF16;
  if (bf && to_fp8)
    hipLaunchKernelGGL((kv_write_kernel<true, true>), grid, block, 0, st, key, value, key_cache,
                       value_cache, slot_mapping, nslots, (int)row, k_scale, v_scale);
  else if (!bf && to_fp8)
    hipLaunchKernelGGL((kv_write_kernel<false, true>), grid, block, 0, st, key, value, key_cache,
                       value_cache, slot_mapping, nslots, (int)row, k_scale, v_scale);
  else
    hipLaunchKernelGGL((kv_write_kernel<true, false>), grid, block, 0, st, key, value, key_cache,
                       value_cache, slot_mapping, nslots, (int)row, k_scale, v_scale);
  return launch_status();
}

// Argument checks shared by the attention entry points.  Returns PKV_OK, an error, or 1 when
// there is nothing to do (no sequences).
static int check_attn(void* out, const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                      int num_seqs, int q_len, int num_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, float scale, int q_dtype, int kv_dtype,
                      float k_scale, float v_scale, int max_context_len, int partition_size,
                      float* tmp_out, float* max_logits, float* exp_sums, int flags) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks < 0 || num_blocks < 0 ||
      max_context_len < 0 || partition_size < -(1 << 20) || q_len < 1 || q_len > kMaxQueryLen)
    return PKV_ERR_SHAPE;
  if ((flags & ~PKV_FLAG_SHARED_BLOCKS) != 0) return PKV_ERR_SHAPE;
  if (num_heads % num_kv_heads != 0 || num_heads / num_kv_heads > 16 || num_kv_heads > 16) return PKV_ERR_SHAPE;
  if ((long long)num_kv_heads * mq_col_blocks(num_heads / num_kv_heads, q_len) > 65535) return PKV_ERR_SHAPE;
  if ((long long)num_seqs * q_len * num_heads >= (1LL << 31)) return PKV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_SHAPE;
  if (block_size < 16 || block_size > 256 || (block_size & (block_size - 1)) != 0) return PKV_ERR_SHAPE;
  if (partition_size > 0 && (partition_size % block_size != 0)) return PKV_ERR_SHAPE;
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (kv_dtype != q_dtype && kv_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (!(std::isfinite(scale) && std::isfinite(k_scale) && std::isfinite(v_scale)))
    return PKV_ERR_SHAPE;
  if (kv_dtype != PKV_FP8_E4M3 && (k_scale != 1.0f || v_scale != 1.0f)) return PKV_ERR_SHAPE;
  if ((long long)max_blocks * block_size > (1LL << 30)) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return 1;
  if (!query || !key_cache || !value_cache || !block_tables || !context_lens) return PKV_ERR_NULL;
  if (num_blocks == 0 || max_blocks == 0) return PKV_ERR_SHAPE;
  if (partition_size == 0 && !out) return PKV_ERR_NULL;
  if (partition_size != 0 && (!tmp_out || !max_logits || !exp_sums)) return PKV_ERR_WORKSPACE;
  if (!aligned(query, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || (out && !aligned(out, 16)) ||
      (tmp_out && !aligned(tmp_out, 16)) || (max_logits && !aligned(max_logits, 4)) ||
      (exp_sums && !aligned(exp_sums, 4)))
    return PKV_ERR_ALIGN;
  if ((long long)num_seqs * ((max_context_len + 15) / 16 + 1) >= (1LL << 31)) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// Checked mode (PKV_CHECK=1): lengths within bounds and every table entry a sequence uses
// inside the pool; with prefix_len > 0 also the shared prefix: the entries covering the first
// min(n, prefix_len) tokens of every row equal row 0's.
static int check_tables(const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                        int num_seqs, int block_size, int num_blocks, int max_context_len,
                        int prefix_len, hipStream_t st) {
  std::vector<int32_t> lens, bt;
  if (!copy_to_host(lens, context_lens, (size_t)num_seqs, st)) return PKV_ERR_LAUNCH;
  if (!copy_to_host(bt, block_tables, (size_t)num_seqs * max_blocks, st)) return PKV_ERR_LAUNCH;
  for (int b = 0; b < num_seqs; ++b) {
    const int n = lens[b];
    if (n < 0 || n > max_context_len || (long long)n > (long long)max_blocks * block_size)
      return PKV_ERR_CHECK;
    for (int j = 0; j < (n + block_size - 1) / block_size; ++j) {
      const int id = bt[(size_t)b * max_blocks + j];
      if (id < 0 || id >= num_blocks) return PKV_ERR_CHECK;
    }
    const int shared = (std::min(n, prefix_len) + block_size - 1) / block_size;
    for (int j = 0; j < shared; ++j)
      if (bt[(size_t)b * max_blocks + j] != bt[j]) return PKV_ERR_CHECK;
  }
  for (int j = 0; j < prefix_len / block_size; ++j)
    if (bt[j] < 0 || bt[j] >= num_blocks) return PKV_ERR_CHECK;
  return PKV_OK;
}

static DecodeParams make_params(void* out, const void* query, const void* key_cache, const void* value_cache,
                                const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                                int num_seqs, int q_len, int num_heads, int num_kv_heads, int block_size,
                                int num_blocks, float scale, float k_scale, float v_scale, int max_context_len,
                                int partition_size, int Pslots, float* tmp_out, float* max_logits,
                                float* exp_sums) {
  DecodeParams p;
  p.B = num_seqs;
  p.L = q_len;
  p.mode = partition_size == 0 ? MODE_SINGLE : (partition_size > 0 ? MODE_FIXED : MODE_BALANCED);
  p.W = partition_size < 0 ? -partition_size : 0;
  // Lengths are clamped to max_context_len, the bound paged_attn_reduce also uses, so both
  // count the same split units; table indices are clamped to the row separately.
  p.cap = max_context_len;
  p.Pslots = Pslots;
  p.out = out;
  p.q = query;
  p.kc = key_cache;
  p.vc = value_cache;
  p.bt = block_tables;
  p.lens = context_lens;
  p.tmp_out = tmp_out;
  p.max_logits = max_logits;
  p.exp_sums = exp_sums;
  p.max_blocks = max_blocks;
  p.Hq = num_heads;
  p.Hkv = num_kv_heads;
  p.G = num_heads / num_kv_heads;
  p.BS = block_size;
  p.num_blocks = num_blocks;
  p.PS = partition_size;
  p.tile_shift = __builtin_ctz((unsigned)block_size) - 4;
  p.c2 = scale * k_scale * kLog2e;
  p.v_scale = v_scale;
  p.t0 = 0;
  p.slot0 = 0;
  p.compact = 0;
  p.knew = nullptr;
  p.vnew = nullptr;
  return p;
}

static void launch_decode_dt(const DecodeParams& p, int head_dim, int q_dtype, int kv_dtype, bool sh, bool last,
                             hipStream_t st) {
  const bool bf = q_dtype == PKV_BF16;
  const bool f8 = kv_dtype == PKV_FP8_E4M3;
  if (p.G * p.L > kDecodeMaxCols) {                        // more columns than a decode wave carries
    if (head_dim == 128) {
      if (f8) { if (bf) launch_mq_tiled<128, KFP8, true>(p, last, st); else launch_mq_tiled<128, KFP8, false>(p, last, st); }
      else    { if (bf) launch_mq_tiled<128, KBF16, true>(p, last, st); else launch_mq_tiled<128, KF16, false>(p, last, st); }
    } else {
      if (f8) { if (bf) launch_mq_tiled<64, KFP8, true>(p, last, st); else launch_mq_tiled<64, KFP8, false>(p, last, st); }
      else    { if (bf) launch_mq_tiled<64, KBF16, true>(p, last, st); else launch_mq_tiled<64, KF16, false>(p, last, st); }
    }
    return;
  }
  if (head_dim == 128) {
    if (f8) { if (bf) launch_decode<128, KFP8, true>(p, sh, last, st); else launch_decode<128, KFP8, false>(p, sh, last, st); }
    else    { if (bf) launch_decode<128, KBF16, true>(p, sh, last, st); else launch_decode<128, KF16, false>(p, sh, last, st); }
  } else {
    if (f8) { if (bf) launch_decode<64, KFP8, true>(p, sh, last, st); else launch_decode<64, KFP8, false>(p, sh, last, st); }
    else    { if (bf) launch_decode<64, KBF16, true>(p, sh, last, st); else launch_decode<64, KF16, false>(p, sh, last, st); }
  }
}

// Shared by paged_attn_decode (q_len 1) and paged_attn_multi_query.
static int attn_entry(void* out, const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                      int num_seqs, int q_len, int num_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, float scale, int q_dtype, int kv_dtype,
                      float k_scale, float v_scale, int max_context_len, int partition_size,
                      float* tmp_out, float* max_logits, float* exp_sums, int flags, void* stream) {
  const TimedCall timed;
  const int rc = check_attn(out, query, key_cache, value_cache, block_tables, max_blocks, context_lens,
                            num_seqs, q_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                            q_dtype, kv_dtype, k_scale, v_scale, max_context_len, partition_size, tmp_out,
                            max_logits, exp_sums, flags);
  if (rc != PKV_OK) return rc > 0 ? PKV_OK : rc;
  const int Pslots = slots_of(max_context_len, partition_size);
  if (partition_size != 0 && Pslots == 0) return PKV_OK;   // every context is empty
  if (partition_size > 0 && Pslots > 65535) return PKV_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (check_mode()) {
    const int cr = check_tables(block_tables, max_blocks, context_lens, num_seqs, block_size, num_blocks,
                                max_context_len, 0, st);
    if (cr != PKV_OK) return cr;
  }
  const DecodeParams p = make_params(out, query, key_cache, value_cache, block_tables, max_blocks, context_lens,
                                     num_seqs, q_len, num_heads, num_kv_heads, block_size, num_blocks, scale,
                                     k_scale, v_scale, max_context_len, partition_size, Pslots, tmp_out,
                                     max_logits, exp_sums);
  launch_decode_dt(p, head_dim, q_dtype, kv_dtype, (flags & PKV_FLAG_SHARED_BLOCKS) != 0, true, st);
  return launch_status();
}

int paged_attn_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                      int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, float scale, int q_dtype, int kv_dtype, float k_scale,
                      float v_scale, int max_context_len, int partition_size, float* tmp_out,
                      float* max_logits, float* exp_sums, int flags, void* stream) {
  return attn_entry(out, query, key_cache, value_cache, block_tables, max_blocks, context_lens, num_seqs, 1,
                    num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, q_dtype, kv_dtype,
                    k_scale, v_scale, max_context_len, partition_size, tmp_out, max_logits, exp_sums, flags,
                    stream);
}

int paged_attn_multi_query(void* out, const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                           int num_seqs, int q_len, int num_heads, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, float scale, int q_dtype, int kv_dtype,
                           float k_scale, float v_scale, int max_context_len, int partition_size,
                           float* tmp_out, float* max_logits, float* exp_sums, int flags, void* stream) {
  return attn_entry(out, query, key_cache, value_cache, block_tables, max_blocks, context_lens, num_seqs,
                    q_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, q_dtype,
                    kv_dtype, k_scale, v_scale, max_context_len, partition_size, tmp_out, max_logits,
                    exp_sums, flags, stream);
}

int paged_attn_decode_noalloc(void* out, const void* query, const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                              int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, float scale, int q_dtype, int kv_dtype, float k_scale,
                              float v_scale, int max_context_len, int partition_size, int flags, void* stream) {
  const TimedCall timed;
  if (partition_size > 0 || partition_size < -(1 << 20)) return PKV_ERR_SHAPE;
  // the argument checks of the single pass (out is always written here)
  const int rc = check_attn(out, query, key_cache, value_cache, block_tables, max_blocks, context_lens, num_seqs,
                            1, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, q_dtype, kv_dtype,
                            k_scale, v_scale, max_context_len, 0, nullptr, nullptr, nullptr, flags);
  if (rc != PKV_OK) return rc > 0 ? PKV_OK : rc;
  hipStream_t st = (hipStream_t)stream;
  const bool sh = (flags & PKV_FLAG_SHARED_BLOCKS) != 0;
  if (partition_size == 0) {                                  // single pass: no partials
    const DecodeParams p = make_params(out, query, key_cache, value_cache, block_tables, max_blocks, context_lens,
                                       num_seqs, 1, num_heads, num_kv_heads, block_size, num_blocks, scale, k_scale,
                                       v_scale, max_context_len, 0, 0, nullptr, nullptr, nullptr);
    launch_decode_dt(p, head_dim, q_dtype, kv_dtype, sh, true, st);
    return launch_status();
  }
  // Balanced split, partials in the compact layout: at most B + Weff - 1 slots per head, where
  // Weff <= min(W, units / kMinChunkTiles) and units <= B * (ceil(max_len / 16) + 1).
  const long long units = (long long)num_seqs * ((max_context_len + 15) / 16 + 1);
  const long long weff = std::max(1LL, std::min((long long)-partition_size, units / kMinChunkTiles));
  const long long rows = (num_seqs + weff - 1) * (long long)num_heads;
  const long long need = rows * (head_dim + 2) * (long long)sizeof(float);
  if (need > (long long)kScratchBytes) return PKV_ERR_SCRATCH;
  void* base = nullptr;
  const int sr = scratch_address(&base);
  if (sr != PKV_OK) return sr;
  float* tmp = (float*)base;                                  // [rows][D], then [rows] twice
  float* ml = tmp + rows * head_dim;
  float* es = ml + rows;
  DecodeParams p = make_params(nullptr, query, key_cache, value_cache, block_tables, max_blocks, context_lens,
                               num_seqs, 1, num_heads, num_kv_heads, block_size, num_blocks, scale, k_scale, v_scale,
                               max_context_len, partition_size, 0, tmp, ml, es);
  p.compact = 1;
  if (max_context_len > 0) launch_decode_dt(p, head_dim, q_dtype, kv_dtype, sh, false, st);
  launch_reduce(out, tmp, ml, es, context_lens, num_seqs, num_heads, head_dim, 1, partition_size, p.cap, 0, 0,
                q_dtype == PKV_BF16, st, 1);
  return launch_status();
}

int paged_attn_decode_append(void* out, const void* query, const void* key, const void* value,
                             void* key_cache, void* value_cache, const int32_t* block_tables, int max_blocks,
                             const int32_t* context_lens, int num_seqs, int num_heads, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, float scale, int dtype,
                             int max_context_len, int partition_size, float* tmp_out, float* max_logits,
                             float* exp_sums, int flags, void* stream) {
  const TimedCall timed;
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_DTYPE;
  const int rc = check_attn(out, query, key_cache, value_cache, block_tables, max_blocks, context_lens,
                            num_seqs, 1, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                            dtype, dtype, 1.f, 1.f, max_context_len, partition_size, tmp_out, max_logits,
                            exp_sums, flags);
  if (rc != PKV_OK) return rc > 0 ? PKV_OK : rc;
  if (!key || !value) return PKV_ERR_NULL;
  if (!aligned(key, 16) || !aligned(value, 16)) return PKV_ERR_ALIGN;
  if ((long long)num_kv_heads * head_dim > (1 << 24)) return PKV_ERR_SHAPE;
  const int Pslots = slots_of(max_context_len, partition_size);
  if (partition_size != 0 && Pslots == 0) return PKV_OK;   // every context is empty: no new token
  if (partition_size > 0 && Pslots > 65535) return PKV_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (check_mode()) {
    const int cr = check_tables(block_tables, max_blocks, context_lens, num_seqs, block_size, num_blocks,
                                max_context_len, 0, st);
    if (cr != PKV_OK) return cr;
  }
  DecodeParams p = make_params(out, query, key_cache, value_cache, block_tables, max_blocks, context_lens,
                               num_seqs, 1, num_heads, num_kv_heads, block_size, num_blocks, scale, 1.f, 1.f,
                               max_context_len, partition_size, Pslots, tmp_out, max_logits, exp_sums);
  const bool sh = (flags & PKV_FLAG_SHARED_BLOCKS) != 0;
  const bool bf = dtype == PKV_BF16;
  if (partition_size < 0) {
    p.knew = key;
    p.vnew = value;
    if (head_dim == 128) {
      if (bf) launch_decode_append<128, KBF16, true>(p, sh, st); else launch_decode_append<128, KF16, false>(p, sh, st);
    } else {
      if (bf) launch_decode_append<64, KBF16, true>(p, sh, st); else launch_decode_append<64, KF16, false>(p, sh, st);
    }
  } else {
    // other schedules: the append scatter, then the decode
    launch(kv_append_kernel, dim3(num_seqs), dim3(256), 0, st, false, key, value, key_cache, value_cache,
           block_tables, context_lens, max_blocks, p.cap, (int)__builtin_ctz((unsigned)block_size), num_blocks,
           num_kv_heads * head_dim);
    launch_decode_dt(p, head_dim, dtype, dtype, sh, true, st);
  }
  return launch_status();
}

int paged_attn_decode_shared_prefix(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables, int max_blocks,
                                    const int32_t* context_lens, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                    float scale, int q_dtype, int kv_dtype, float k_scale, float v_scale,
                                    int max_context_len, int prefix_len, int prefix_partition_size,
                                    int partition_size, float* tmp_out, float* max_logits, float* exp_sums,
                                    int flags, void* stream) {
  const TimedCall timed;
  if (partition_size >= 0) return PKV_ERR_SHAPE;              // the suffix runs the balanced split
  const int rc = check_attn(out, query, key_cache, value_cache, block_tables, max_blocks, context_lens,
                            num_seqs, 1, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                            q_dtype, kv_dtype, k_scale, v_scale, max_context_len, partition_size, tmp_out,
                            max_logits, exp_sums, flags);
  if (rc != PKV_OK) return rc > 0 ? PKV_OK : rc;
  if (!out) return PKV_ERR_NULL;
  if (prefix_len < 0 || prefix_len % block_size != 0 || (long long)prefix_len > (long long)max_blocks * block_size)
    return PKV_ERR_SHAPE;
  if (prefix_len > 0 && (prefix_partition_size < 16 || prefix_partition_size % 16 != 0))
    return PKV_ERR_SHAPE;
  const int parts = prefix_parts(prefix_len, prefix_partition_size);
  const int Pslots = shared_prefix_slots(max_context_len, prefix_len, prefix_partition_size, partition_size);
  if (Pslots > 65535) return PKV_ERR_SHAPE;
  const long long prefix_groups = ((long long)num_seqs * (num_heads / num_kv_heads) + kPrefixCols - 1) /
                                  kPrefixCols * ((num_kv_heads * (long long)parts + 7) / 8 * 8);
  if (prefix_groups >= (1LL << 31)) return PKV_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (check_mode()) {
    const int cr = check_tables(block_tables, max_blocks, context_lens, num_seqs, block_size, num_blocks,
                                max_context_len, prefix_len, st);
    if (cr != PKV_OK) return cr;
  }
  DecodeParams p = make_params(nullptr, query, key_cache, value_cache, block_tables, max_blocks, context_lens,
                               num_seqs, 1, num_heads, num_kv_heads, block_size, num_blocks, scale, k_scale,
                               v_scale, max_context_len, partition_size, Pslots, tmp_out, max_logits, exp_sums);
  p.t0 = prefix_len / 16;
  p.slot0 = parts;
  const bool bf = q_dtype == PKV_BF16;
  const bool f8 = kv_dtype == PKV_FP8_E4M3;
  if (parts > 0) {
    PrefixParams pp;
    pp.q = query;
    pp.kc = key_cache;
    pp.vc = value_cache;
    pp.bt = block_tables;
    pp.lens = context_lens;
    pp.tmp_out = tmp_out;
    pp.max_logits = max_logits;
    pp.exp_sums = exp_sums;
    pp.B = num_seqs;
    pp.Hq = num_heads;
    pp.Hkv = num_kv_heads;
    pp.G = num_heads / num_kv_heads;
    pp.num_blocks = num_blocks;
    pp.cap = p.cap;
    pp.max_blocks = max_blocks;
    pp.bs_shift = __builtin_ctz((unsigned)block_size);
    pp.prefix_len = prefix_len;
    pp.chunk = prefix_partition_size;
    pp.parts = parts;
    pp.hp8 = (num_kv_heads * parts + 7) / 8 * 8;
    pp.Pslots = Pslots;
    pp.c2 = p.c2;
    pp.v_scale = v_scale;
    if (head_dim == 128) {
      if (f8) { if (bf) launch_prefix<128, KFP8, true>(pp, st); else launch_prefix<128, KFP8, false>(pp, st); }
      else    { if (bf) launch_prefix<128, KBF16, true>(pp, st); else launch_prefix<128, KF16, false>(pp, st); }
    } else {
      if (f8) { if (bf) launch_prefix<64, KFP8, true>(pp, st); else launch_prefix<64, KFP8, false>(pp, st); }
      else    { if (bf) launch_prefix<64, KBF16, true>(pp, st); else launch_prefix<64, KF16, false>(pp, st); }
    }
  }
  if (Pslots > parts)
    launch_decode_dt(p, head_dim, q_dtype, kv_dtype, (flags & PKV_FLAG_SHARED_BLOCKS) != 0, false, st);
  launch_reduce(out, tmp_out, max_logits, exp_sums, context_lens, num_seqs, num_heads, head_dim, Pslots,
                partition_size, p.cap, p.t0, parts, bf, st);
  return launch_status();
}

int paged_attn_shared_prefix_slots(int max_context_len, int prefix_len, int prefix_partition_size,
                                   int partition_size) {
  if (max_context_len < 0 || prefix_len < 0 || partition_size >= 0 ||
      (prefix_len > 0 && prefix_partition_size <= 0))
    return PKV_ERR_SHAPE;
  return shared_prefix_slots(max_context_len, prefix_len, prefix_partition_size, partition_size);
}

int paged_attn_multi_query_split(int num_heads, int num_kv_heads, int head_dim, int q_len, int q_dtype,
                                 int kv_dtype) {
  if (num_heads <= 0 || num_kv_heads <= 0 || num_kv_heads > 16 || num_heads % num_kv_heads != 0 || q_len < 1 ||
      q_len > kMaxQueryLen || (head_dim != 64 && head_dim != 128))
    return 0;
  const int G = num_heads / num_kv_heads;
  if (G * q_len <= kDecodeMaxCols) return paged_attn_balanced_split(num_kv_heads, head_dim, q_dtype, kv_dtype);
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  // fill every compute unit once: W ranges x Hkv heads x column blocks tiled workgroups
  const bool bf = q_dtype == PKV_BF16, f8 = kv_dtype == PKV_FP8_E4M3;
  int occ;
  if (head_dim == 128)
    occ = f8 ? (bf ? mq_occupancy<128, KFP8, true>() : mq_occupancy<128, KFP8, false>())
             : (bf ? mq_occupancy<128, KBF16, true>() : mq_occupancy<128, KF16, false>());
  else
    occ = f8 ? (bf ? mq_occupancy<64, KFP8, true>() : mq_occupancy<64, KFP8, false>())
             : (bf ? mq_occupancy<64, KBF16, true>() : mq_occupancy<64, KF16, false>());
  const long long per_w = (long long)num_kv_heads * mq_col_blocks(G, q_len);
  const long long w = (long long)prop.multiProcessorCount * occ / per_w;
  return -(int)(w > 0 ? w : 1);
}

int paged_attn_prefix_split(int num_seqs, int num_heads, int num_kv_heads, int prefix_len) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || prefix_len <= 0)
    return 0;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  const long long cols = (long long)num_seqs * (num_heads / num_kv_heads);
  const long long units = (cols + kPrefixCols - 1) / kPrefixCols * num_kv_heads;
  long long parts = (prop.multiProcessorCount + units - 1) / units;
  if (parts < 1) parts = 1;
  long long size = (prefix_len + parts - 1) / parts;
  size = (size + kStage - 1) / kStage * kStage;
  return (int)size;
}

int paged_attn_reduce(void* out, const float* tmp_out, const float* max_logits, const float* exp_sums,
                      const int32_t* context_lens, int num_seqs, int num_heads, int head_dim,
                      int max_context_len, int partition_size, int out_dtype, void* stream) {
  const TimedCall timed;
  if (num_seqs < 0 || num_heads <= 0 || max_context_len < 0 || partition_size == 0 ||
      partition_size < -(1 << 20))
    return PKV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_SHAPE;
  if (out_dtype != PKV_F16 && out_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !context_lens) return PKV_ERR_NULL;
  const int Pslots = slots_of(max_context_len, partition_size);
  if (Pslots > 0 && (!tmp_out || !max_logits || !exp_sums)) return PKV_ERR_WORKSPACE;
  if (!aligned(out, 16) || (tmp_out && !aligned(tmp_out, 16)) || !aligned(context_lens, 4))
    return PKV_ERR_ALIGN;
  if (Pslots > 65535 || (long long)num_seqs * num_heads >= (1LL << 31)) return PKV_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  if (check_mode()) {
    std::vector<int32_t> lens;
    if (!copy_to_host(lens, context_lens, (size_t)num_seqs, st)) return PKV_ERR_LAUNCH;
    for (int n : lens)
      if (n < 0 || n > max_context_len) return PKV_ERR_CHECK;
  }
  launch_reduce(out, tmp_out, max_logits, exp_sums, context_lens, num_seqs, num_heads, head_dim, Pslots,
                partition_size, max_context_len, 0, 0, out_dtype == PKV_BF16, st);
  return launch_status();
}

}  // extern "C"
