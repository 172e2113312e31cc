// bi_lmhead.hip - the lm_head projection on the CDNA4 matrix cores, fused with
// the per-token statistics of each vocabulary tile, so the [N, V] logits never
// reach HBM, and with the gradient of those logits for the backward.  C ABI:
// bi_lmhead_tile_stats, bi_lmhead_grad_logits, bi_lmhead_tiles,
// bi_lmhead_tile_rows (include/bi_logprob.h); bi_stats_combine finishes the
// statistics and bi_lmhead_backward (bi_lmhead_bwd.hip) the backward.
//
// What is computed: the chunked lm_head of "ZeroSyncGRPOTrainer" (logits of a
// vocabulary slice from the hidden states and the replicated projection, bf16
// products accumulated in fp32), reduced at once to the shard-local statistics
// of "[RL] Avoid full-vocab gather for TP policy statistics" (torchtitan PR
// #4685), Why: local max, softmax denominator, target logit and the
// entropy-weighted sum.  How it is computed is this file's own design:
//
//  * D[v][n] = sum_k W[v, k] H[n, k] with v_mfma_f32_32x32x16_bf16, A = lm_head
//    rows, B = hidden rows.  Lane l of a 32 x 32 block holds token l % 32 and
//    vocabulary rows 8*(r/4) + 4*(l/32) + r%4 of accumulator r, so a token's
//    statistics need no shuffle inside a block.
//  * A workgroup of 8 waves (2 per SIMD, one workgroup per CU) owns a
//    256-vocab x 256-token tile: 2 (vocab) x 4 (tokens) waves, each a
//    128 x 64 part (4 x 2 blocks, 128 accumulators).  The 256 x 256 tile keeps
//    the operand bytes streamed from L2 per MFMA at their minimum for what the
//    register file can hold.
//  * K runs in stages of 64, each stage two 32 KB units (its 256 W rows, its
//    256 H rows) streamed through a FIFO of five LDS slots (all 160 KB).
//    Units are filled straight from global memory (global_load_lds_dwordx4,
//    no register staging).  A stage is 4 MFMA K steps; each step's MFMAs are
//    issued one by one with the next step's fragment reads between them.
//    Before the last step each wave waits for its own requests of stage s+1
//    and for its LDS reads of stage s, and the one barrier per stage both
//    publishes stage s+1 and frees stage s's slots.  Stage s+2's H unit is
//    then requested between the last step's MFMAs, and its W unit, which
//    has a stage longer to land, between the next stage's first steps: the
//    requests never arrive in one burst that would hold up the MFMAs queued
//    behind them.  The loop body has no branch; the last stages, whose
//    refills would lie past the end, run in a separate tail loop.  (Four
//    slots, a 2-deep ring of whole stages, remain a build option.)
//  * LDS rows are 128 bytes (8 chunks of 8 bf16).  Chunk c of row r is stored
//    in slot c ^ g(r), g(r) = (r ^ ((r >> 3) & 3)) & 7, which puts the 8- and
//    16-lane groups of every ds_read_b128 on distinct banks.  The shape knobs
//    below also build 64-byte-row variants.
//  * Rows past the end of W or H are read clamped to the last row (never out
//    of bounds); their logits are masked to -inf / their tokens not written.
//  * Each logit is the same MFMA sequence over K whatever n_tokens is, and the
//    statistics of a tile are folded in a fixed order (the lane's 64 values,
//    then the lane halves, then the two vocabulary waves), so the result of a
//    token is batch-invariant bit for bit.
//  * Tiles are visited XCD-aware: workgroup b runs on XCD b % 8, and each XCD
//    takes a contiguous range of tiles in which 8 token tiles sweep the
//    vocabulary tiles together, so concurrent tiles share W and H slices in
//    that XCD's L2.

#include <type_traits>

#include "bi_common.h"

namespace {

using namespace bi_internal;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tuning knobs (shape of the pipeline only; every choice computes the same
// statistics tile of 256 vocabulary rows, bit for bit).
#ifndef BI_LM_SLOTS
#define BI_LM_SLOTS 5      // LDS slots of one operand's stage: 5, or 4 (two whole stages)
#endif
#ifndef BI_LM_GROUP
#define BI_LM_GROUP 8      // token tiles that sweep the vocabulary together
#endif
#ifndef BI_LM_BK
#define BI_LM_BK 64        // K per LDS stage: 64 (128-byte row slices) or 32 (64-byte)
#endif
#ifndef BI_LM_WAVES
#define BI_LM_WAVES 8      // waves per workgroup: 2 (vocab) x 4 (tokens) or 2 x 2
#endif

constexpr int kTV = 256;                  // vocab rows per tile (= per statistics tile)
constexpr int kTN = kTV;                  // tokens per tile
constexpr int kWaves = BI_LM_WAVES;
constexpr int kWT = kWaves / 2;           // token waves (vocab waves: 2)
constexpr int kWV = kTV / 2;              // vocab rows per wave
constexpr int kWN = kTN / kWT;            // tokens per wave
constexpr int kXB = kWV / 32;             // 32-row MFMA blocks per wave: vocab
constexpr int kYB = kWN / 32;             //                             tokens
constexpr int kBK = BI_LM_BK;             // K per LDS stage
constexpr int kKS = kBK / 16;             // MFMA K steps per stage
constexpr int kChunks = kBK / 8;          // 16-byte chunks per row slice
constexpr int kBlockRows = 1024 / (kBK * 2);   // rows per 1 KB fill block
constexpr int kSlots = BI_LM_SLOTS;       // LDS slots, one operand's stage each
constexpr int kThreads = 64 * kWaves;
constexpr int kRowBytes = kBK * 2;        // bytes per row per stage
constexpr int kUnitBytes = kTV * kRowBytes;   // one operand's rows of one stage
constexpr int kRingBytes = kSlots * kUnitBytes;
constexpr int kLoadsU = kUnitBytes / (kThreads * 16);       // requests per lane per unit
constexpr int kLoads = 2 * kLoadsU;                         // per lane per stage
constexpr int kGroup = BI_LM_GROUP;       // token tiles that sweep together

static_assert(kUnitBytes % (kThreads * 16) == 0, "fill split");
static_assert(kBK == 32 || kBK == 64, "stage depth");
static_assert(kSlots >= 4 && (kSlots - 2) * kLoadsU < 64, "ring depth");
static_assert(kRingBytes <= 160 * 1024, "LDS size");
static_assert(kWaves == 4 || kWaves == 8, "waves");
static_assert(kWN % 32 == 0, "wave tile");
static_assert(kXB * kYB >= kXB + kYB, "one fragment read per MFMA");
// waves per SIMD: eight-wave workgroups need ~210 registers a wave (two waves
// a SIMD); four-wave ones run two workgroups a CU when the LDS allows
constexpr int kWGsPerCU = (160 * 1024) / kRingBytes;
constexpr int kWavesPerEU = kWaves == 8 ? 2 : (kWGsPerCU >= 2 ? 2 : 1);

struct LmArgs {
  const uint16_t* hidden;   // [n_tok, ldh] bf16 bits
  const uint16_t* weight;   // [n_voc, ldw] bf16 bits
  int64_t n_tok, n_voc, d, ldh, ldw;
  int64_t vocab_offset, vocab;
  const int64_t* labels;
  int64_t ignore_index;
  bi_stats* stats;          // [tiles_v][n_tok]          (statistics kernel)
  int32_t* status_flag;
  int64_t tiles_v, tiles_n;
  const float* lse;         // [n_tok]                   (grad-logits kernel)
  const float* token_weights;   // [n_tok] or NULL (= 1)
  uint16_t* gout;           // [n_voc, ldg] bf16 bits: gradient of the logits, vocabulary-major
  int64_t ldg;
  void* dout;               // [n_voc, ldd] fp32 or bf16: the product itself (product kernels)
  int64_t ldd;
  int dout_bf16;
  int64_t gpad;             // grad-logits kernel: rows n_voc .. gpad-1 of gout written as zeros
  int64_t tpad;             //                     and columns n_tok .. tpad-1 of every row
  int64_t kvalid_h;         // transposed product: rows of the H-side operand that exist
};

// What a workgroup does with its fp32 tile of D = W . H^T:
//   kModeStats     per-token statistics of each 256-row vocabulary tile;
//   kModeGrad      the gradient of the logits, bf16, vocabulary-major;
//   kModeProductT  D added into an fp32 output, operands with M (N) contiguous:
//                  "W" is stored [K][n_voc] and "H" [K][n_tok];
//   kModeProductNT D itself, fp32 or bf16, "W" with K contiguous ([n_voc][K])
//                  and "H" stored [K][n_tok].
enum { kModeStats = 0, kModeGrad = 1, kModeProductT = 3, kModeProductNT = 4 };

// Whether the "W" (A) and "H" (B) operands of a mode are stored [K][columns]
// (read with transposing LDS reads) rather than with K contiguous.
template <int MODE> constexpr bool kTransW = MODE == kModeProductT;
template <int MODE> constexpr bool kTransH = MODE == kModeProductT || MODE == kModeProductNT;

// Tile (tv, tn) of linear tile index t: groups of kGroup token tiles sweep
// the vocabulary tiles together.
__device__ inline void lm_tile_at(const LmArgs& p, int64_t t, int64_t* tv, int64_t* tn) {
  const int64_t group = t / (kGroup * p.tiles_v), r = t % (kGroup * p.tiles_v);
  const int64_t rows_in_group = min(int64_t(kGroup), p.tiles_n - group * kGroup);
  *tn = group * kGroup + r % rows_in_group;
  *tv = r / rows_in_group;
}

// Tile of workgroup b: workgroup b runs on XCD b % 8, and each XCD takes a
// contiguous range of linear tile indices.  False for padding workgroups.
__device__ inline bool lm_tile_of(const LmArgs& p, int64_t b, int64_t* tv, int64_t* tn) {
  const int64_t total = p.tiles_v * p.tiles_n;
  const int64_t per_xcd = (total + 7) / 8;
  const int64_t t = (b % 8) * per_xcd + b / 8;
  if (t >= total) return false;
  lm_tile_at(p, t, tv, tn);
  return true;
}

// Slot of a row's 16-byte chunks in LDS: chunk c of row r sits in slot
// c ^ lm_swz(r).  It depends only on r mod 32 (so it is the same for every
// 32-row MFMA block) and makes the 8- and 16-lane groups of a ds_read_b128
// (rows r0 .. r0+7 or r0+15, one chunk each) hit distinct bank groups.
__device__ inline int lm_swz(int r) {
  if constexpr (kChunks == 4) return ((r >> 1) ^ (r >> 2)) & 3;   // 64-byte rows
  else return (r ^ ((r >> 3) & 3)) & 7;                          // 128-byte rows
}

// s_waitcnt on the vector-memory and LDS counters (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 left at its maximum, lgkmcnt 11:8)
template <int VM, int LGKM>
__device__ inline void wait_counts() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "waitcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// Workgroup barrier that orders LDS traffic in the compiler but adds no wait
// of its own (the waits are explicit).
__device__ inline void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void lds_void;

// The K loop streams units: unit 2s holds stage s's 256 W rows (kBK wide),
// unit 2s+1 its 256 H rows, and unit u lands in LDS slot u % kSlots.  With
// four slots that is a ring of two whole stages; a fifth slot lets every
// stage's W unit be requested a stage earlier, so 1.5 stages are in flight
// instead of one.  This lane's part of filling one unit: kLoadsU requests,
// each 16 bytes of global memory into 16 bytes of a 1 KB block that the wave
// writes contiguously (lane order); block q of the slot holds kBlockRows
// rows.  Request i reads row row0 + kBlockRows*kWaves*i of the operand,
// clamped to the tile's last valid row, at the chunk that its LDS position
// holds; the tile bases are uniform (SGPRs) and the lane's offset is 32-bit.
struct LmFill {
  const char* wbase;   // W row v0 (transposed: K-row 0, column v0)
  const char* hbase;   // H row n0 (transposed: K-row 0, column n0)
  uint32_t ldw2, ldh2; // row pitches in bytes
  int wlast, hlast;    // last valid operand row within the tile
  int row0;            // this lane's first row
  int trow0;           // transposed side: this lane's first K-row of a stage
  uint32_t cbytes;     // byte offset of the chunk this lane's slot holds
  uint32_t lds0;       // this wave's first block: wave * 1 KB
  uint32_t wc, hc;     // transposed: the lane's chunk offset, clamped per side
  int64_t wklast, hklast;   // transposed: last K-row that exists, per side
};

// A pointer that is the same in every lane, marked so for the compiler (the
// fill's scalar-base operand needs it in SGPRs).
__device__ inline const char* uniform_ptr(const char* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
}

// Transposed operands (both of kModeProductT, the H side of kModeProductNT)
// are stored [K][columns]: a unit holds
// the stage's 64 K-rows of the tile's 256 columns, 512 bytes each, and the
// 16-byte chunk c of K-row k sits in chunk c ^ lm_swz_t(k).  A wave's request
// covers two K-rows (1 KB); request i of a lane reads K-row
// trow0 + 2 kWaves i of the stage, clamped to the last K-row that exists, at
// the chunk its LDS position holds, clamped to the last chunk with columns in
// the tile (so nothing is read past a row's end; the columns past the tile's
// end are never stored).
constexpr int kTRowBytes = kTV * 2;
static_assert(kBK * kTRowBytes == kUnitBytes, "transposed unit = one stage's K-rows");
__device__ inline int lm_swz_t(int k) { return 4 * (k & 3); }

template <int MODE>
__device__ inline LmFill lm_fill_setup(const LmArgs& p, int64_t v0, int64_t n0, int wave,
                                       int lane) {
  LmFill f{};
  // K-contiguous side: 1 KB blocks of kBlockRows rows; transposed side: a
  // wave's request covers two K-rows
  const int rb = lane / kChunks, slot = lane % kChunks;
  f.row0 = kBlockRows * wave + rb;
  f.cbytes = uint32_t(16 * (slot ^ lm_swz(f.row0)));   // lm_swz(row0 + 64 i) == lm_swz(row0)
  f.trow0 = 2 * wave + (lane >> 5);
  const int lc = (lane & 31) ^ lm_swz_t(f.trow0);     // lm_swz_t(trow0 + 2 kWaves i) == lm_swz_t(trow0)
  f.ldw2 = uint32_t(p.ldw * 2);
  f.ldh2 = uint32_t(p.ldh * 2);
  f.lds0 = uint32_t(wave) * 1024u;
  if constexpr (kTransW<MODE>) {
    f.wc = uint32_t(16 * min(lc, int((min(p.n_voc - v0, int64_t(kTV)) - 1) >> 3)));
    f.wbase = uniform_ptr(reinterpret_cast<const char*>(p.weight + v0));
    f.wklast = p.d - 1;
  } else {
    f.wbase = uniform_ptr(reinterpret_cast<const char*>(p.weight + v0 * p.ldw));
    f.wlast = int(min(p.n_voc - v0, int64_t(kTV)) - 1);
  }
  if constexpr (kTransH<MODE>) {
    f.hc = uint32_t(16 * min(lc, int((min(p.n_tok - n0, int64_t(kTN)) - 1) >> 3)));
    f.hbase = uniform_ptr(reinterpret_cast<const char*>(p.hidden + n0));
    f.hklast = p.kvalid_h - 1;
  } else {
    f.hbase = uniform_ptr(reinterpret_cast<const char*>(p.hidden + n0 * p.ldh));
    f.hlast = int(min(p.n_tok - n0, int64_t(kTN)) - 1);
  }
  return f;
}

static_assert((kBlockRows * kWaves) % 32 == 0, "a lane's rows share one swizzle");

// LDS byte address of a pointer into shared memory.
__device__ inline uint32_t lds_addr(const char* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// Request i of one unit: operand W (is_w) or H, K stage `stage`, into the
// slot at LDS address `slot`.  The byte offset from the tile's base fits 31
// bits: row <= 255, the row pitch is at most 2^23 bytes and stage * kRowBytes
// below 2^23 (the entry points cap d and the strides at 2^22 elements).
// Written as inline assembly so that the compiler does not track these LDS
// writes: it would otherwise wait for every request in flight before any LDS
// read.  The waits are explicit instead (wait_counts before each barrier);
// the compiler's own vmcnt waits stay correct, since extra requests only make
// them stricter.  The LDS-DMA load reads M0, which the compiler writes just
// before the asm with a scalar instruction: one wait state (s_nop 0) must
// separate the two.
// (Transposed: the stage's K-row 0 is the uniform base, so the offset is at
// most 63 pitches plus 512 bytes.)
template <int MODE>
__device__ inline void lm_fill1(const LmFill& f, uint32_t slot, int stage, bool is_w, int i) {
  const char* base;
  uint32_t off;
  if (is_w ? kTransW<MODE> : kTransH<MODE>) {
    const int64_t k0 = int64_t(stage) * kBK;
    const uint32_t pitch = is_w ? f.ldw2 : f.ldh2;
    const int lim = int(min((is_w ? f.wklast : f.hklast) - k0, int64_t(kBK - 1)));
    const int kr = min(f.trow0 + 2 * kWaves * i, lim);
    base = uniform_ptr((is_w ? f.wbase : f.hbase) + k0 * pitch);
    off = uint32_t(kr) * pitch + (is_w ? f.wc : f.hc);
  } else {
    const int row = min(f.row0 + kBlockRows * kWaves * i, is_w ? f.wlast : f.hlast);
    base = is_w ? f.wbase : f.hbase;
    off = uint32_t(row) * (is_w ? f.ldw2 : f.ldh2) + f.cbytes + uint32_t(stage) * kRowBytes;
  }
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "{m0}"(slot + f.lds0 + uint32_t(kWaves * i) * 1024u)
               : "memory");
}

// Request i of unit u (0 <= i < kLoadsU) into the ring at LDS address `ring`;
// units past the last stage (u >= 2 ns) are not requested.
template <int MODE>
__device__ inline void lm_fill_unit1(const LmFill& f, uint32_t ring, int u, int ns, int i) {
  if ((u >> 1) < ns)
    lm_fill1<MODE>(f, ring + uint32_t(u % kSlots) * kUnitBytes, u >> 1, (u & 1) == 0, i);
}

// Wait until at most n of this wave's newest units are still in flight
// (0 <= n <= kSlots - 2; requests complete in order) and its LDS reads are done.
__device__ inline void wait_units(int n) {
  static_assert(kSlots <= 5, "wait_units covers n <= 3");
  switch (n) {
    case 0: wait_counts<0, 0>(); break;
    case 1: wait_counts<kLoadsU, 0>(); break;
    case 2: wait_counts<2 * kLoadsU, 0>(); break;
    default: wait_counts<3 * kLoadsU, 0>(); break;
  }
}

struct LmFrag {
  bf16x8 a[kXB], b[kYB];
};

// The lane's fragment offsets within a unit.  K-major operands: the 16 bytes
// of each K step (row lr of the wave's first block, chunk 2 kk + half).
// Transposed operands: for block x (y), the 8 bytes this lane supplies to a
// transposing read of K-rows 0..3 of the step (the reads of K-rows 4..7 and of
// later steps are fixed distances on).
struct LmOffs {
  uint32_t w[kKS], h[kKS];
  uint32_t tw[kXB], th[kYB];
};

template <int MODE>
__device__ inline LmOffs lm_offsets(int wv, int wt, int lane) {
  LmOffs o{};
  const int lr = lane & 31, half = lane >> 5;
  if constexpr (kTransW<MODE> || kTransH<MODE>) {
    // ds_read_b64_tr_b16: within each 16-lane group, lane i receives the
    // 16-bit element i % 4 of the 8 bytes that lanes i / 4, 4 + i / 4,
    // 8 + i / 4 and 12 + i / 4 supply.  Lane 4e + q of group g supplies K-row
    // e (+8 for groups 2 and 3) at columns 4q .. 4q+3 (+16 for groups 1 and
    // 3) of the block, so lane l receives column l % 32 at K 8 (l / 32) + 0..3:
    // the MFMA operand's layout.  The K-row's swizzle is lm_swz_t(e).
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    const uint32_t lane_off = uint32_t((8 * (g >> 1) + e) * kTRowBytes + 8 * (q & 1));
    const int cl = 2 * (g & 1) + (q >> 1);   // chunk within the block's four
#pragma unroll
    for (int x = 0; x < kXB; ++x)
      o.tw[x] = lane_off + uint32_t(16 * ((((kWV * wv + 32 * x) >> 3) ^ lm_swz_t(e)) + cl));
#pragma unroll
    for (int y = 0; y < kYB; ++y)
      o.th[y] = lane_off + uint32_t(16 * ((((kWN * wt + 32 * y) >> 3) ^ lm_swz_t(e)) + cl));
  }
  if constexpr (!kTransW<MODE> || !kTransH<MODE>) {
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      const uint32_t in_row = uint32_t(lr * kRowBytes + 16 * ((2 * kk + half) ^ lm_swz(lr)));
      o.w[kk] = uint32_t(kWV * wv * kRowBytes) + in_row;
      o.h[kk] = uint32_t(kWN * wt * kRowBytes) + in_row;
    }
  }
  return o;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// K-rows 0..7 of a transposed fragment: two transposing reads 4 K-rows apart
__device__ inline bf16x8 lm_read_t(const char* p) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * kTRowBytes));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Operand fragment j of K step kk of the stage whose W and H units are in
// the slots w and h, in the order the step's MFMAs first use them (A0,
// B0 .. B(kYB-1), A1 ..).
template <int MODE>
__device__ inline void lm_read1(LmFrag& fr, const char* w, const char* h, const LmOffs& o,
                                int kk, int j) {
  const int kbytes = 16 * kk * kTRowBytes;
  if (j >= 1 && j <= kYB) {
    if constexpr (kTransH<MODE>)
      fr.b[j - 1] = lm_read_t(h + o.th[j - 1] + kbytes);
    else
      fr.b[j - 1] = *reinterpret_cast<const bf16x8*>(h + o.h[kk] + (j - 1) * 32 * kRowBytes);
  } else {
    const int x = j == 0 ? 0 : j - kYB;
    if constexpr (kTransW<MODE>)
      fr.a[x] = lm_read_t(w + o.tw[x] + kbytes);
    else
      fr.a[x] = *reinterpret_cast<const bf16x8*>(w + o.w[kk] + x * 32 * kRowBytes);
  }
}

template <int MODE>
__device__ inline void lm_read(LmFrag& fr, const char* w, const char* h, const LmOffs& o,
                               int kk) {
#pragma unroll
  for (int j = 0; j < kXB + kYB; ++j) lm_read1<MODE>(fr, w, h, o, kk, j);
}

constexpr int kMfmas = kXB * kYB;                      // MFMAs per wave per K step
constexpr int kFillsPerMfma = (kLoads + kMfmas - 1) / kMfmas;

// The MFMAs of one K step (fragments `cur`), each followed by `extra(m)`: the
// reads and requests that the step overlaps are issued one by one between
// the MFMAs, so the matrix pipe never waits for a burst of them.  The
// scheduling barriers keep exactly this order.
template <typename Extra>
__device__ inline void lm_mma_with(const LmFrag& cur, f32x16 (&acc)[kXB][kYB], Extra&& extra) {
#pragma unroll
  for (int m = 0; m < kMfmas; ++m) {
    const int x = m / kYB, y = m % kYB;
    acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[x], cur.b[y], acc[x][y], 0, 0, 0);
    extra(m);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// (m, c, S, U, t) of one token: a (+) b with a taken first
__device__ inline void lm_merge(Acc& a, float& ta, const Acc& b, float tb) {
  const float M = fmaxf(a.m, b.m);
  const float C = ref_of(M);
  Acc x = a, y = b;
  rebase(x, C);
  rebase(y, C);
  a.m = M;
  a.c = C;
  a.S = x.S + y.S;
  a.U = x.U + y.U;
  ta = ta + tb;
}

// Statistics of each token over one tile's 256 vocabulary rows, written as
// the tile's bi_stats (fixed order: the lane's values, the lane halves, the
// two vocabulary waves).
__device__ inline void lm_stats_epilogue(const LmArgs& p, f32x16 (&acc)[kXB][kYB],
                                         const int64_t (&lab)[kYB], int64_t tv, int64_t tn,
                                         int wv, int wt, int lr, int half,
                                         float (&red)[kWT][kYB][32][4]) {
  const int64_t v0 = tv * kTV, n0 = tn * kTN;
  const int64_t wrow0 = v0 + kWV * wv;     // first vocabulary row of this wave
  // rows of this wave that exist (uniform); on the ragged last tile the
  // others are masked to -inf first, so that full tiles select nothing
  const int valid = int(max(int64_t(0), min(p.n_voc - wrow0, int64_t(kWV))));
  if (valid < kWV) {
#pragma unroll
    for (int x = 0; x < kXB; ++x)
#pragma unroll
      for (int y = 0; y < kYB; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * x + 8 * (r >> 2) + 4 * half + (r & 3);   // within the wave
          if (row >= valid) acc[x][y][r] = -INFINITY;
        }
  }
  float tl[kYB];
  Acc lo[kYB];
#pragma unroll
  for (int y = 0; y < kYB; ++y) {
    float z[16 * kXB];
#pragma unroll
    for (int x = 0; x < kXB; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) z[16 * x + r] = acc[x][y][r];
    Acc a = acc_empty();
    accumulate<8, 2 * kXB>(a, z);
    // the label's logit, held by exactly one lane of one vocabulary wave (if
    // here); the select chain runs only when some lane of the wave needs it
    float t = 0.0f;
    const bool bad = lab[y] != p.ignore_index && (lab[y] < 0 || lab[y] >= p.vocab);
    const int64_t yl = lab[y] - p.vocab_offset - wrow0;   // row within this wave's 128
    const bool mine = !bad && lab[y] != p.ignore_index && lab[y] - p.vocab_offset < p.n_voc &&
                      yl >= 0 && yl < kWV && half == ((yl >> 2) & 1);
    if (__builtin_amdgcn_ballot_w64(mine)) {
      const int q = mine ? int(yl >> 5) * 16 + int((yl & 31) >> 3) * 4 + int(yl & 3) : -1;
#pragma unroll
      for (int k = 0; k < 16 * kXB; ++k) t = q == k ? z[k] : t;
    }
    // lane halves (same token, other rows), lower half first
    Acc o;
    o.m = __shfl_xor(a.m, 32);
    o.c = __shfl_xor(a.c, 32);
    o.S = __shfl_xor(a.S, 32);
    o.U = __shfl_xor(a.U, 32);
    const float ot = __shfl_xor(t, 32);
    Acc l = half ? o : a, h = half ? a : o;
    float tlo = half ? ot : t, thi = half ? t : ot;
    lm_merge(l, tlo, h, thi);
    lo[y] = l;
    tl[y] = tlo;
    if (wv == 1 && half == 0) {
      red[wt][y][lr][0] = l.m;
      red[wt][y][lr][1] = l.S;
      red[wt][y][lr][2] = l.U;
      red[wt][y][lr][3] = tlo;
    }
  }
  wait_counts<63, 0>();   // this wave's LDS writes are done
  lds_barrier();
  if (wv == 0 && half == 0) {
#pragma unroll
    for (int y = 0; y < kYB; ++y) {
      const int64_t j = n0 + kWN * wt + 32 * y + lr;
      Acc b;
      b.m = red[wt][y][lr][0];
      b.c = ref_of(b.m);
      b.S = red[wt][y][lr][1];
      b.U = red[wt][y][lr][2];
      Acc a = lo[y];
      float t = tl[y];
      lm_merge(a, t, b, red[wt][y][lr][3]);
      if (j < p.n_tok) {
        const bool bad = lab[y] != p.ignore_index && (lab[y] < 0 || lab[y] >= p.vocab);
        const float d = fmaf(a.m, kLog2e, a.c);
        const float f = exp2_hw(-d);
        bi_stats out;
        out.max = a.m;
        out.sumexp = a.S == 0.0f ? 0.0f : a.S * f;
        out.sumexp_logit = a.S == 0.0f ? 0.0f : kLn2 * (fmaf(-d, a.S, a.U) * f);
        out.target = bad ? NAN : t;
        p.stats[tv * p.n_tok + j] = out;
        if (bad && p.status_flag) atomicOr(p.status_flag, BI_FLAG_BAD_LABEL);
      }
    }
  }
}

// Byte offset of (vocabulary row, token) in the gradient epilogue's LDS tile,
// bf16 [kTV][kTN]: the 16-byte chunks of a row are XOR-swizzled by 4 * (row
// bit 0 + 2 * row bit 2), so the rows r, r+1, r+4, r+5 that one 4-byte write
// instruction covers land on disjoint banks.
__device__ inline int lm_grad_at(int row, int tok) {
  const int key = ((row & 1) | ((row >> 1) & 2)) << 2;
  return row * (kTN * 2) + (((tok >> 3) ^ key) << 4) + ((tok & 7) << 1);
}

// two floats as bf16 (round to nearest even), `lo` in the low half
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {__bf16(lo), __bf16(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// kModeStats:   per-token statistics of each 256-row vocabulary tile.
// kModeGrad:    the gradient of the logits, w * (softmax - onehot) from the
//               saved lse, written as bf16 (the cross-entropy backward of PR
//               #4685 Summary, on the lm_head logits).
// kModeProductT: the product of two operands stored [K][columns], added into
//               an fp32 output: the lm_head backward's grad_hidden += G . W_c
//               with G vocabulary-major and the lm_head rows as they are.
// kModeProductNT: the product of one operand with K-contiguous rows and one
//               stored [K][columns], written fp32 or bf16 (RNE): the lm_head
//               backward's grad_W_c = G_c^T . hidden with G's rows (tokens
//               contiguous) and the hidden states as they are.
// Same main loop in every mode; the operands stored [K][columns] are read
// with transposing LDS reads.
template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU, kWavesPerEU)))
void lmhead_kernel(LmArgs p) {
  __shared__ __attribute__((aligned(1024))) char ring[kRingBytes];
  int64_t tv, tn;
  if (!lm_tile_of(p, blockIdx.x, &tv, &tn)) return;   // whole workgroup exits together
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave & 1, wt = wave >> 1;
  const int64_t v0 = tv * kTV, n0 = tn * kTN;
  const int lr = lane & 31, half = lane >> 5;

  // the labels of this lane's tokens (and for the gradient their lse and
  // weight), fetched early: the epilogue uses them once the K loop is done
  int64_t lab[kYB];
  float tlse[kYB], tw[kYB];
#pragma unroll
  for (int y = 0; y < kYB; ++y) {
    const int64_t j = n0 + kWN * wt + 32 * y + lr;
    const bool in = j < p.n_tok;
    if constexpr (MODE == kModeStats || MODE == kModeGrad)
      lab[y] = in ? p.labels[j] : p.ignore_index;
    if constexpr (MODE == kModeGrad) {
      tlse[y] = in ? p.lse[j] : 0.0f;
      tw[y] = in && p.token_weights ? p.token_weights[j] : 1.0f;
    }
  }

  const LmFill fill = lm_fill_setup<MODE>(p, v0, n0, wave, lane);
  const int ns = int(p.d / kBK);

  const LmOffs offs = lm_offsets<MODE>(wv, wt, lane);

  f32x16 acc[kXB][kYB];
#pragma unroll
  for (int x = 0; x < kXB; ++x)
#pragma unroll
    for (int y = 0; y < kYB; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.0f;

  // With five slots the W unit of stage s+2 (unit 2s+4) is requested during
  // stage s's first kKS-1 steps, a few requests per step, instead of right
  // after a barrier: only stage s+2's H unit goes out then.  (All waves
  // requesting a whole stage at once after each barrier holds up the MFMAs
  // that are ordered after those requests.)
  constexpr bool kSpread = kSlots == 5;
  constexpr int kPrologue = kSpread ? kSlots - 1 : kSlots;

  // prologue: units 0 .. kPrologue-1 requested, stage 0 (units 0 and 1)
  // landed and visible
  const uint32_t rbase = lds_addr(ring);
#pragma unroll
  for (int u = 0; u < kPrologue; ++u)
#pragma unroll
    for (int i = 0; i < kLoadsU; ++i) lm_fill_unit1<MODE>(fill, rbase, u, ns, i);
  wait_units(min(kPrologue, 2 * ns) - 2);   // units 2 .. min(kPrologue, 2 ns) - 1 may fly on
  lds_barrier();
  LmFrag fr[2];
  lm_read<MODE>(fr[0], ring, ring + kUnitBytes, offs, 0);

  // Stage s from the slots of units 2s (W) and 2s+1 (H), K step kk's
  // fragments in fr[kk & 1]: the next step's fragments are read while this
  // step's MFMAs run.  Before the last step's MFMAs: stage s+1 must have
  // landed (this wave's requests: all but the units requested after unit
  // 2s+3, at most kSlots-4 of them; the barrier covers the other waves'),
  // and this wave's reads of stage s must be done; after the barrier stage
  // s+1 is visible and stage s's two slots are free for units 2s+kSlots and
  // 2s+kSlots+1, whose requests are spread over the last step.  Those units
  // exist (stage < ns) for every stage but the last kTail ones: the stages
  // before them run without a branch (TAIL = false), the last ones check.
  constexpr int kTail = (kSlots + 1) / 2;
  int sw = 0;   // slot of stage s's W unit; its H unit is in the next slot
  auto stage = [&](int s, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    const int sh = sw + 1 == kSlots ? 0 : sw + 1;
    const int nw = sh + 1 == kSlots ? 0 : sh + 1;   // stage s+1's slots
    const int nh = nw + 1 == kSlots ? 0 : nw + 1;
    const char* wbuf = ring + sw * kUnitBytes;
    const char* hbuf = ring + sh * kUnitBytes;
    // spread: unit 2s+4 (W of stage s+2) into the slot before sw, freed at
    // the previous barrier
    const uint32_t fp = rbase + uint32_t(sw == 0 ? kSlots - 1 : sw - 1) * kUnitBytes;
    const bool pending = !TAIL || s + 2 < ns;
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      LmFrag& now = fr[kk & 1];
      LmFrag& next = fr[(kk + 1) & 1];
      if (kk + 1 < kKS) {
        lm_mma_with(now, acc, [&](int m) {
          if (m < kXB + kYB) lm_read1<MODE>(next, wbuf, hbuf, offs, kk + 1, m);
          if constexpr (kSpread) {
            // request r goes out in step r (kKS-1) / kLoadsU, after the step's reads
#pragma unroll
            for (int r = 0; r < kLoadsU; ++r)
              if (r * (kKS - 1) / kLoadsU == kk &&
                  m == kXB + kYB + r - (kk * kLoadsU + kKS - 2) / (kKS - 1) && pending)
                lm_fill1<MODE>(fill, fp, s + 2, true, r);
          }
        });
      } else {
        // units requested so far: 0 .. min(2s + kSlots, 2ns) - 1
        if (TAIL) wait_units(max(0, min(2 * s + kSlots, 2 * ns) - (2 * s + 4)));
        else wait_counts<(kSlots - 4) * kLoadsU, 0>();
        lds_barrier();
        // unit 2s+kSlots into slot sw, unit 2s+kSlots+1 into slot sh
        const uint32_t fa = rbase + uint32_t(sw) * kUnitBytes;
        const uint32_t fb = rbase + uint32_t(sh) * kUnitBytes;
        const int sa = s + kSlots / 2, sb = s + (kSlots + 1) / 2;
        const char* nwbuf = ring + nw * kUnitBytes;
        const char* nhbuf = ring + nh * kUnitBytes;
        lm_mma_with(now, acc, [&](int m) {
          if constexpr (kSpread) {
            // only unit 2s+5 (H of stage s+2) now, every other MFMA; unit
            // 2s+6 is the next stage's spread W unit
            if (m % 2 == 0 && m / 2 < kLoadsU && (!TAIL || sa < ns))
              lm_fill1<MODE>(fill, fa, sa, false, m / 2);
          } else {
#pragma unroll
            for (int q = 0; q < kFillsPerMfma; ++q) {
              const int r = m * kFillsPerMfma + q;
              if (r < kLoadsU) {
                if (!TAIL || sa < ns) lm_fill1<MODE>(fill, fa, sa, kSlots % 2 == 0, r);
              } else if (r < kLoads) {
                if (!TAIL || sb < ns) lm_fill1<MODE>(fill, fb, sb, kSlots % 2 == 1, r - kLoadsU);
              }
            }
          }
          if (m < kXB + kYB) lm_read1<MODE>(next, nwbuf, nhbuf, offs, 0, m);
        });
      }
    }
    sw = nw;
  };
  int s = 0;
  for (; s < ns - kTail; ++s) stage(s, std::false_type());
  for (; s < ns; ++s) stage(s, std::true_type());
  wait_counts<0, 15>();   // no request may still be writing LDS when the workgroup ends
  lds_barrier();          // every wave is done with the ring: the epilogues reuse it

  if constexpr (MODE == kModeProductT) {
    // D[i][j] += the tile, fp32, for the rows and columns that exist (the
    // W side's columns are D's rows); for a given accumulator register the 64
    // lanes cover 32 consecutive columns of 2 rows
    float* dout = static_cast<float*>(p.dout);
#pragma unroll
    for (int x = 0; x < kXB; ++x)
#pragma unroll
      for (int y = 0; y < kYB; ++y) {
        const int64_t j = n0 + kWN * wt + 32 * y + lr;
        if (j >= p.n_tok) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t i = v0 + kWV * wv + 32 * x + 8 * (r >> 2) + 4 * half + (r & 3);
          if (i < p.n_voc) dout[i * p.ldd + j] += acc[x][y][r];
        }
      }
  } else if constexpr (MODE == kModeProductNT) {
    // D[i][j] for the rows and columns that exist; for a given accumulator
    // register the 64 lanes cover 32 consecutive columns of 2 rows
#pragma unroll
    for (int x = 0; x < kXB; ++x)
#pragma unroll
      for (int y = 0; y < kYB; ++y) {
        const int64_t j = n0 + kWN * wt + 32 * y + lr;
        if (j >= p.n_tok) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t i = v0 + kWV * wv + 32 * x + 8 * (r >> 2) + 4 * half + (r & 3);
          if (i >= p.n_voc) continue;
          if (p.dout_bf16)
            static_cast<__bf16*>(p.dout)[i * p.ldd + j] = __bf16(acc[x][y][r]);
          else
            static_cast<float*>(p.dout)[i * p.ldd + j] = acc[x][y][r];
        }
      }
  } else if constexpr (MODE == kModeGrad) {
    // gradient of the logits: w * (p - [v == y]), p = 2^((z - lse) * log2e)
    // as the row backward computes it; +0 for ignored tokens, NaN for bad
    // labels.  The tile goes through LDS (the ring is free now) as bf16
    // [vocab row][token], so that it leaves as whole 16-byte vectors of 8
    // tokens: vocabulary-major.  A lane holds 4 consecutive rows of one
    // token; neighbouring lanes (tokens t, t+1) swap halves of their packed
    // row pairs, so each lane writes 4-byte words of two tokens (even lane:
    // rows 0 and 2 of the four, odd lane: rows 1 and 3).  16-byte chunks of a
    // row are XOR-swizzled by row bits 0 and 2, which makes the four rows of
    // one write instruction fall on different banks.  Every element is
    // written as w * p first; the label's element, w * (p - 1), afterwards by
    // the lane holding its logit (same wave, so in order).
    static_assert(kTV * kTN * 2 <= kRingBytes, "grad tile fits the ring");
    const int odd = lr & 1;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;   // v_perm: see below
#pragma unroll
    for (int y = 0; y < kYB; ++y) {
      const int tok = kWN * wt + 32 * y + lr;   // token within the tile
      const int64_t lb = lab[y];                // tokens past the end: ignored, never stored
      const bool ignored = lb == p.ignore_index;
      const bool bad = !ignored && (lb < 0 || lb >= p.vocab);
      const float lse = tlse[y];
      const float wg = bad ? NAN : tw[y];
      // halves of a packed word belong to tokens tp and tp+1: keep each one
      // unless its token is ignored (+0 whatever its logits)
      const uint32_t keep = ignored ? 0u : 0xffffu;
      const uint32_t keep_nb = uint32_t(__builtin_amdgcn_mov_dpp(int(keep), 0xB1, 0xF, 0xF, true));
      const uint32_t mask = odd ? (keep_nb | (keep << 16)) : (keep | (keep_nb << 16));
      const int tp = tok & ~1;
#pragma unroll
      for (int x = 0; x < kXB; ++x)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float gv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) gv[i] = wg * exp2_hw((acc[x][y][4 * g + i] - lse) * kLog2e);
          // rows r0..r3 of token t packed in pairs (low half the lower row)
          const uint32_t p01 = pack_bf16(gv[0], gv[1]), p23 = pack_bf16(gv[2], gv[3]);
          // the neighbour's (token t ^ 1), by a quad permutation [1, 0, 3, 2]
          const uint32_t q01 = uint32_t(__builtin_amdgcn_mov_dpp(int(p01), 0xB1, 0xF, 0xF, true));
          const uint32_t q23 = uint32_t(__builtin_amdgcn_mov_dpp(int(p23), 0xB1, 0xF, 0xF, true));
          // v_perm picks bytes of {q (bytes 4-7), p (bytes 0-3)}: an even lane
          // keeps the low halves (its row r0 / r2: tokens t, t+1), an odd lane
          // the high ones (r1 / r3: tokens t-1, t)
          const uint32_t a = __builtin_amdgcn_perm(q01, p01, sel) & mask;
          const uint32_t b = __builtin_amdgcn_perm(q23, p23, sel) & mask;
          const int row = kWV * wv + 32 * x + 8 * g + 4 * half + odd;
          *reinterpret_cast<uint32_t*>(ring + lm_grad_at(row, tp)) = a;
          *reinterpret_cast<uint32_t*>(ring + lm_grad_at(row + 2, tp)) = b;
        }
      // the label's element, if this wave holds it: the select chain runs
      // only when some lane of the wave needs it
      const int64_t yl = lb - p.vocab_offset - v0 - kWV * wv;   // row within this wave's 128
      const bool mine = !ignored && !bad && yl >= 0 && yl < kWV && half == ((yl >> 2) & 1);
      if (__builtin_amdgcn_ballot_w64(mine)) {
        const int q = mine ? int(yl >> 5) * 16 + int((yl & 31) >> 3) * 4 + int(yl & 3) : -1;
        float z = 0.0f;
#pragma unroll
        for (int k = 0; k < 16 * kXB; ++k) z = q == k ? acc[k / 16][y][k % 16] : z;
        if (mine) {
          const float pr = exp2_hw((z - lse) * kLog2e);
          *reinterpret_cast<__bf16*>(ring + lm_grad_at(kWV * wv + int(yl), tok)) =
              __bf16(tw[y] * (pr - 1.0f));
        }
      }
      if (bad && p.status_flag && tv == 0 && wv == 0 && half == 0)
        atomicOr(p.status_flag, BI_FLAG_BAD_LABEL);
    }
    wait_counts<63, 0>();
    lds_barrier();
    // rows v0 .. v0+255, 16-byte chunks of 8 tokens; 32 threads per row.
    // Rows n_voc .. gpad-1 and columns n_tok .. tpad-1 (the lm_head backward
    // pads its chunk to whole K stages both ways) are written as zeros: the
    // tile holds +0 for tokens past the end, which count as ignored, and
    // tpad - 1 lies in the last token tile.
    const bool vec = (p.ldg % 8) == 0 && (reinterpret_cast<uintptr_t>(p.gout) % 16) == 0;
    constexpr int kChunksPerRow = kTN / 8;
#pragma unroll 4
    for (int q = tid; q < kTV * kChunksPerRow; q += kThreads) {
      const int row = q / kChunksPerRow, c = q % kChunksPerRow;
      const int64_t i = v0 + row, j0 = n0 + 8 * c;
      if (i >= p.gpad || j0 >= p.tpad) continue;
      u32x4 v = *reinterpret_cast<const u32x4*>(ring + lm_grad_at(row, 8 * c));
      if (i >= p.n_voc) v = u32x4{0u, 0u, 0u, 0u};
      uint16_t* dst = p.gout + i * p.ldg + j0;
      if (vec && j0 + 8 <= p.tpad) {
        // non-temporal: G is read back only by the next kernels, long after
        // this tile's operand lines have left L2
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
      } else {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        for (int e = 0; e < 8 && j0 + e < p.tpad; ++e)
          dst[e] = uint16_t(w4[e >> 1] >> (16 * (e & 1)));
      }
    }
  } else {
    typedef float Red[kWT][kYB][32][4];
    static_assert(sizeof(Red) <= kRingBytes, "reduction fits the ring");
    lm_stats_epilogue(p, acc, lab, tv, tn, wv, wt, lr, half, *reinterpret_cast<Red*>(ring));
  }
}

// Shared validation of the lm_head entry points; fills the common arguments.
int lm_setup(const char* fn, LmArgs* a, const void* hidden, const void* weight, int64_t n_tokens,
             int64_t n_vocab_rows, int64_t d, int64_t hidden_stride, int64_t weight_stride,
             int64_t vocab_offset, int64_t vocab, const int64_t* labels, int64_t ignore_index,
             int32_t* status_flag) {
  if (n_tokens < 0 || n_vocab_rows < 0) return fail(BI_ERR_SHAPE, "%s: negative size", fn);
  if (d < kBK || d % kBK != 0 || d > (int64_t(1) << 22))
    return fail(BI_ERR_SHAPE, "%s: d = %lld must be a positive multiple of %d (at most 2^22)",
                fn, (long long)d, kBK);
  if (hidden_stride < d || weight_stride < d || hidden_stride % 8 || weight_stride % 8 ||
      hidden_stride > (int64_t(1) << 22) || weight_stride > (int64_t(1) << 22))
    return fail(BI_ERR_SHAPE, "%s: strides must be >= d, multiples of 8 and at most 2^22 elements",
                fn);
  if (vocab < 1 || vocab_offset < 0 || vocab_offset + n_vocab_rows > vocab)
    return fail(BI_ERR_SHAPE, "%s: rows [%lld, %lld) outside the vocabulary [0, %lld)", fn,
                (long long)vocab_offset, (long long)(vocab_offset + n_vocab_rows),
                (long long)vocab);
  if (n_tokens == 0 || n_vocab_rows == 0) return BI_OK;
  if (!hidden || !weight || !labels)
    return fail(BI_ERR_NULL, "%s: hidden, weight and labels are required", fn);
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(labels, 8) ||
      !aligned(status_flag, 4))
    return fail(BI_ERR_ALIGN, "%s: hidden and weight need 16-byte alignment", fn);
  a->hidden = static_cast<const uint16_t*>(hidden);
  a->weight = static_cast<const uint16_t*>(weight);
  a->n_tok = n_tokens;
  a->n_voc = n_vocab_rows;
  a->d = d;
  a->ldh = hidden_stride;
  a->ldw = weight_stride;
  a->vocab_offset = vocab_offset;
  a->vocab = vocab;
  a->labels = labels;
  a->ignore_index = ignore_index;
  a->status_flag = status_flag;
  a->tiles_v = (n_vocab_rows + kTV - 1) / kTV;
  a->tiles_n = (n_tokens + kTN - 1) / kTN;
  return BI_OK;
}

template <int MODE>
int lm_launch(const char* fn, const LmArgs& a, bi_stream_t stream) {
  const int64_t total = a.tiles_v * a.tiles_n;
  int64_t blocks = 8 * ((total + 7) / 8);
  if (blocks > 0x7fffffff) return fail(BI_ERR_SHAPE, "%s: too many tiles", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(lmhead_kernel<MODE>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, a);
  return launched(fn);
}

}  // namespace


extern "C" {

int64_t bi_lmhead_tile_rows(void) { return kTV; }

int64_t bi_lmhead_tiles(int64_t n_vocab_rows) {
  return n_vocab_rows <= 0 ? 0 : (n_vocab_rows + kTV - 1) / kTV;
}

int bi_lmhead_tile_stats(const void* hidden, const void* weight, int64_t n_tokens,
                         int64_t n_vocab_rows, int64_t d, int64_t hidden_stride,
                         int64_t weight_stride, int64_t vocab_offset, int64_t vocab,
                         const int64_t* labels, int64_t ignore_index, bi_stats* stats,
                         int32_t* status_flag, bi_stream_t stream) {
  const char* fn = "bi_lmhead_tile_stats";
  LmArgs a{};
  if (int r = lm_setup(fn, &a, hidden, weight, n_tokens, n_vocab_rows, d, hidden_stride,
                       weight_stride, vocab_offset, vocab, labels, ignore_index, status_flag))
    return r;
  if (n_tokens == 0 || n_vocab_rows == 0) return ok();
  if (!stats) return fail(BI_ERR_NULL, "%s: stats is required", fn);
  if (!aligned(stats, 16)) return fail(BI_ERR_ALIGN, "%s: stats needs 16-byte alignment", fn);
  a.stats = stats;
  return lm_launch<kModeStats>(fn, a, stream);
}

int bi_lmhead_grad_logits(const void* hidden, const void* weight, int64_t n_tokens,
                          int64_t n_vocab_rows, int64_t d, int64_t hidden_stride,
                          int64_t weight_stride, int64_t vocab_offset, int64_t vocab,
                          const int64_t* labels, int64_t ignore_index, const float* lse,
                          const float* token_weights, void* grad_logits, int64_t grad_stride,
                          int32_t* status_flag, bi_stream_t stream) {
  return lmhead_grad_logits_padded("bi_lmhead_grad_logits", hidden, weight, n_tokens,
                                   n_vocab_rows, d, hidden_stride, weight_stride, vocab_offset,
                                   vocab, labels, ignore_index, lse, token_weights, grad_logits,
                                   grad_stride, n_vocab_rows, n_tokens, status_flag, stream);
}

}  // extern "C"

namespace bi_internal {

int lmhead_grad_logits_padded(const char* fn, const void* hidden, const void* weight,
                              int64_t n_tokens, int64_t n_vocab_rows, int64_t d,
                              int64_t hidden_stride, int64_t weight_stride, int64_t vocab_offset,
                              int64_t vocab, const int64_t* labels, int64_t ignore_index,
                              const float* lse, const float* token_weights, void* grad_logits,
                              int64_t grad_stride, int64_t pad_rows, int64_t pad_cols,
                              int32_t* status_flag, bi_stream_t stream) {
  if (pad_rows < n_vocab_rows || pad_rows > (n_vocab_rows + kTV - 1) / kTV * kTV)
    return fail(BI_ERR_SHAPE, "%s: padded rows outside the last tile", fn);
  LmArgs a{};
  if (int r = lm_setup(fn, &a, hidden, weight, n_tokens, n_vocab_rows, d, hidden_stride,
                       weight_stride, vocab_offset, vocab, labels, ignore_index, status_flag))
    return r;
  if (grad_stride < n_tokens)
    return fail(BI_ERR_SHAPE, "%s: grad_stride %lld < n_tokens %lld", fn, (long long)grad_stride,
                (long long)n_tokens);
  if (pad_cols < n_tokens || pad_cols > (n_tokens + kTN - 1) / kTN * kTN ||
      pad_cols > grad_stride)
    return fail(BI_ERR_SHAPE, "%s: padded columns outside the last tile or the row", fn);
  if (n_tokens == 0 || n_vocab_rows == 0) return ok();
  if (!lse || !grad_logits) return fail(BI_ERR_NULL, "%s: lse and grad_logits are required", fn);
  if (!aligned(lse, 4) || !aligned(token_weights, 4) || !aligned(grad_logits, 2))
    return fail(BI_ERR_ALIGN, "%s: misaligned pointer", fn);
  a.lse = lse;
  a.token_weights = token_weights;
  a.gout = static_cast<uint16_t*>(grad_logits);
  a.ldg = grad_stride;
  a.gpad = pad_rows;
  a.tpad = pad_cols;
  return lm_launch<kModeGrad>(fn, a, stream);
}

// D[i][j] = sum_k A[i][k] B[k][j]: A [m][k] bf16 with rows of k contiguous
// elements (its columns from kvalid_b on must be zero), B [k][n] bf16 with
// rows of n contiguous elements of which only the first kvalid_b exist (the
// rest read as row kvalid_b - 1); D fp32 or bf16 (RNE), overwritten.
int lmhead_product_nt(const char* fn, const void* a, int64_t m, int64_t lda, const void* b,
                      int64_t n, int64_t ldb, int64_t k, int64_t kvalid_b, void* d, int64_t ldd,
                      bool d_bf16, bi_stream_t stream) {
  if (k < kBK || k % kBK != 0 || k > (int64_t(1) << 22) || kvalid_b < 1 || kvalid_b > k ||
      kvalid_b <= k - kBK || lda < k || ldb < n || lda % 8 || ldb % 8 ||
      lda > (int64_t(1) << 22) || ldb > (int64_t(1) << 22) || ldd < n || m > 0x7fffffff ||
      n > 0x7fffffff)
    return fail(BI_ERR_SHAPE, "%s: product shape outside the kernel's limits", fn);
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, d_bf16 ? 2 : 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned product operand", fn);
  if (m == 0 || n == 0) return BI_OK;
  LmArgs p{};
  p.weight = static_cast<const uint16_t*>(a);
  p.hidden = static_cast<const uint16_t*>(b);
  p.n_voc = m;
  p.n_tok = n;
  p.d = k;
  p.ldw = lda;
  p.ldh = ldb;
  p.kvalid_h = kvalid_b;
  p.dout = d;
  p.ldd = ldd;
  p.dout_bf16 = d_bf16 ? 1 : 0;
  p.tiles_v = (m + kTV - 1) / kTV;
  p.tiles_n = (n + kTN - 1) / kTN;
  return lm_launch<kModeProductNT>(fn, p, stream);
}

// D[i][j] += sum_k A[k][i] B[k][j]: A [k][m] and B [k][n] bf16 with rows of
// m (n) contiguous elements, of which B has only its first kvalid_b rows
// (the rest read as row kvalid_b - 1; A's rows there must be zero); D fp32.
int lmhead_product_t(const char* fn, const void* a, int64_t m, int64_t lda, const void* b,
                     int64_t n, int64_t ldb, int64_t k, int64_t kvalid_b, float* d, int64_t ldd,
                     bi_stream_t stream) {
  if (k < kBK || k % kBK != 0 || k > (int64_t(1) << 31) - kBK || kvalid_b < 1 ||
      kvalid_b > k || kvalid_b <= k - kBK || lda < m || ldb < n || lda % 8 || ldb % 8 ||
      lda > (int64_t(1) << 22) || ldb > (int64_t(1) << 22) || ldd < n || m > 0x7fffffff ||
      n > 0x7fffffff)
    return fail(BI_ERR_SHAPE, "%s: transposed product shape outside the kernel's limits", fn);
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 4))
    return fail(BI_ERR_ALIGN, "%s: misaligned product operand", fn);
  if (m == 0 || n == 0) return BI_OK;
  LmArgs p{};
  p.weight = static_cast<const uint16_t*>(a);
  p.hidden = static_cast<const uint16_t*>(b);
  p.n_voc = m;
  p.n_tok = n;
  p.d = k;
  p.ldw = lda;
  p.ldh = ldb;
  p.kvalid_h = kvalid_b;
  p.dout = d;
  p.ldd = ldd;
  p.tiles_v = (m + kTV - 1) / kTV;
  p.tiles_n = (n + kTN - 1) / kTN;
  return lm_launch<kModeProductT>(fn, p, stream);
}

}  // namespace bi_internal
