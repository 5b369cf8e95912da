// mkv_partial_mfma.hip -- matrix-core partial-attention kernels for gfx950.
//
// Minima-KV's format-specific kernels compute partial attention states over
// the pages of one format, read in place without a dense shadow (arXiv
// 2608.23834, page 1, Abstract).  Here both formats run on the CDNA4 matrix
// cores with fp32 accumulation:
//
//  * Work item = (layer, chunk of pages, KV head); a workgroup of 4 waves
//    takes one item, wave w the pages w, w+4, ...; each KV page is read once
//    for the whole GQA group, copied HBM -> LDS by LDS-DMA loads a few units
//    ahead of use.  The 4 wave states are merged in LDS and one partial
//    (m, l, acc) per item is written.
//  * Scores S^T = K Q^T with v_mfma_f32_16x16x32_f16: A = 16 tokens x 32
//    channels of K, B = 32 channels x 16 query rows.  Query rows 0..G-1 hold
//    fp16(q) and rows 8..8+G-1 the fp16 remainder q - fp16(q), so one DPP
//    row-rotate by 8 adds the two halves (q carried to ~22 bits).  For TQ3
//    each MFMA covers exactly one 32-channel scale group and the fp32 group
//    scale multiplies its result; codes enter the MFMA as exact fp16 u, and
//    the -4 offset of every group arrives as one more MFMA per page (token
//    scales x per-group sums of q) that seeds the scores.
//  * Online softmax in log2 units with a lazy rescale: the running max moves
//    only when a page's max exceeds it by more than 15 (p <= 2^15, finite in
//    fp16).
//  * P V: A = P (rows 0..G-1 fp16(p), rows 8..8+G-1 the remainder).  TQ3 V
//    is u * s split into an exact fp16 pair hi + lo; one
//    v_mfma_f32_16x16x32_f16 per 16-channel tile takes both, its k index
//    running over (token, part) with P repeated for the two parts.  The -4
//    offset is W = sum_t P s (one v_mfma_f32_16x16x16_f16 per page), taken
//    off as O - 4 W when the item ends.  FP8 V is exact in fp16
//    (v_mfma_f32_16x16x16_f16, k = the page's 16 tokens).
//  Lane maps follow the byte layout in mkv_format.h: a TQ3 lane's triples
//  arrive in one aligned chunk, and each run of 4 triples becomes 32 fp16
//  codes through one FP6 conversion (decode32 below).
//  Rotated TQ3 pages (a layer with a sign vector: the stale pages hold the
//  codes of c H (signs . x), H the Sylvester-Hadamard matrix) run in their
//  own kernel instance (ROT): its TQ3 items read queries rotated by
//  rotate_q_kernel, q' = H (signs . q) / (c d), so the scores are unchanged,
//  and rotate each partial state back, signs . (H acc) / (c d), before
//  storing it.  Plain layers run the ROT = false instances, compiled as before.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kItemWaves;
constexpr int kThreads = 64 * kWaves;

// Item trace (measurement support): a build with -DMKV_ITEM_TRACE=1, made
// into its own library, records per workgroup the constant 100 MHz clock
// (s_memrealtime) at points of its work item: slot 0 at entry, 1 once the
// query fragments are built, 2 once the partial state is stored, 3 the item
// (pages | tq3 << 32 | KV head << 40 | request << 48), 4 + w when wave w's
// first page has landed, 16 + w when wave w leaves its page loop (the last
// item of a workgroup that runs several).  mkv_debug_item_trace reads it back.
// The product build compiles none of it.
#ifndef MKV_ITEM_TRACE
#define MKV_ITEM_TRACE 0
#endif
constexpr bool kItemTrace = MKV_ITEM_TRACE != 0;
__device__ uint64_t g_item_trace[kItemTrace ? kTraceBlocks * kTraceSlots : 1];
// every lane of the calling wave stores the same word (wave-uniform callers)
__device__ inline void trace_mark(int slot, uint64_t value) {
  if constexpr (kItemTrace) g_item_trace[(blockIdx.x % kTraceBlocks) * kTraceSlots + slot] = value;
}
__device__ inline void trace_time(int slot) {
  if constexpr (kItemTrace) trace_mark(slot, __builtin_amdgcn_s_memrealtime());
}
__device__ inline bool wave0() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0; }
// The running max moves only when a page's max exceeds it by more than
// kRescale (log2 units), so p <= 2^15 stays finite in fp16.
constexpr float kRescale = 15.0f;
constexpr int kNoMask = 1 << 20;

__device__ inline h2 u2h(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ inline uint32_t h2u(h2 h) { return __builtin_bit_cast(uint32_t, h); }

// {x[l], x[l ^ 32]} and {x[l], x[l ^ 16]} (in either order) with one VALU
// permute (gfx950 v_permlane32_swap / v_permlane16_swap): reductions over the
// four 16-lane rows without an LDS round trip.
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max of four scores (finite or -inf: arithmetic results, so no signalling
// NaN to quiet and no canonicalising moves)
__device__ inline float max4(float a, float b, float c, float d) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3\n\tv_max_f32 %0, %0, %4" : "=&v"(r) : "v"(a), "v"(b), "v"(c), "v"(d));
  return r;
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float dpp_ror8(float x) {             // lane l <- lane (l ^ 8) within each 16-lane row
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
}

typedef uint32_t u6 __attribute__((ext_vector_type(6)));
typedef _Float16 h32 __attribute__((ext_vector_type(32)));
typedef uint32_t u16v __attribute__((ext_vector_type(16)));

// V codes of a 12-byte block (4 triples = 32 codes, code k of the stream at
// bits [3k, 3k + 3), little endian) -> 32 fp16 codes u, exact (normal fp16,
// which the V scales multiply exactly into hi + lo pairs).  Read as 6-bit
// fields, the stream holds two codes per field.  With the high code masked
// away a field is an E2M3 value with zero exponent bits, i.e. the subnormal
// u / 8, and gfx950 converts 32 such fields in one instruction (scale 8 makes
// them u).  The high codes take a second pass over the stream shifted down by
// 3 bits.  Element i < 16 is the low code of field i (slot 2 (i % 4) of triple
// i / 4), element 16 + i the high code (slot 2 (i % 4) + 1).
__device__ inline h32 decode32(uint32_t w0, uint32_t w1, uint32_t w2) {
  // low 3 bits of every 6-bit field; the pattern repeats every 3 words
  constexpr uint32_t M0 = 0xC71C71C7u, M1 = 0x71C71C71u, M2 = 0x1C71C71Cu;
  u6 f;
  f[0] = w0 & M0;
  f[1] = w1 & M1;
  f[2] = w2 & M2;
  f[3] = __builtin_amdgcn_alignbit(w1, w0, 3) & M0;
  f[4] = __builtin_amdgcn_alignbit(w2, w1, 3) & M1;
  f[5] = (w2 >> 3) & M2;                  // M2 keeps bits <= 28: nothing comes from a next word
  return __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(f, 8.0f);
}

// K codes of a 12-byte block (w0..w2, 16 six-bit fields, mkv_format.h)
// straight into MFMA operands, with shifts and masks only.  Window q of the
// block is the block shifted right by 6 f0 - 4 bits, f0 the first field of
// fields f0 and f0 + 2, f0 = 0, 1, 4, 5, 8, 9, 12, 13 for q = 0..7; in it the
// low code of field f0 sits at bits 4..6, that of f0 + 2 at 16..18, and their
// high codes at 7..9 and 19..21.  Masked (kLoCodes, kHiCodes), a window is
// two fp16 values of one scale group: u 2^(s - 24) with s the code's bit
// position in its half (subnormals, which the matrix cores take exactly).
// Windows 0..3 with kLoCodes hold group 4b of the block, 4..7 group 4b + 1;
// with kHiCodes, 4b + 2 and 4b + 3.  An operand of 4 windows lists the
// group's channels (of the lane's 8) in the order tq3_channel gives.
constexpr uint32_t kLoCodes = 0x00070070u;
constexpr uint32_t kHiCodes = 0x00380380u;
__device__ inline void code_windows(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t (&x)[8]) {
  x[0] = w0 << 4;                                   // fields 0, 2
  x[1] = w0 >> 2;                                   // 1, 3
  x[2] = __builtin_amdgcn_alignbit(w1, w0, 20);     // 4, 6
  x[3] = __builtin_amdgcn_alignbit(w1, w0, 26);     // 5, 7
  x[4] = __builtin_amdgcn_alignbit(w2, w1, 12);     // 8, 10
  x[5] = __builtin_amdgcn_alignbit(w2, w1, 18);     // 9, 11
  x[6] = w2 >> 4;                                   // 12, 14
  x[7] = w2 >> 10;                                  // 13, 15
}
// fp16 element k (0..7) of a 4-window operand: channel of the lane's 8
// (field f0 + (k & 1) * 2 of window k / 2) and the bit position of its code
// (low codes at 4 / 0 in the low / high half, high codes at 7 / 3)
__host__ __device__ constexpr int tq3_channel(int k) { return (k & ~3) + ((k >> 1) & 1) + 2 * (k & 1); }
__host__ __device__ constexpr int tq3_code_shift(bool hi_codes, int k) { return (hi_codes ? 3 : 0) + ((k & 1) ? 0 : 4); }
static_assert(tq3_channel(0) == 0 && tq3_channel(1) == 2 && tq3_channel(2) == 1 && tq3_channel(3) == 3 &&
              tq3_channel(4) == 4 && tq3_channel(5) == 6 && tq3_channel(6) == 5 && tq3_channel(7) == 7,
              "windows hold fields (0, 2), (1, 3), (4, 6), (5, 7)");

typedef __attribute__((address_space(3))) void lds_void;
// Page lists and chunk tables are read-only during the launch: read them
// through the constant address space so the (wave-uniform) loads go to the
// scalar unit and never count against the vector-memory counter that the
// staging waits below rely on.
typedef const __attribute__((address_space(4))) int32_t* cptr_i32;
typedef int i16v __attribute__((ext_vector_type(16)));
typedef const __attribute__((address_space(4))) i16v* cptr_i16;

// Per-head-dim constants and the LDS plan of a 12-wave workgroup (one per CU):
//   [ring: 12 waves x kWaveRing3 bytes][sq: score-MFMA B operands, NG x 64 x 16 B]
//   [per-wave query-row maxima]
// (135 KB at d = 256).  A wave's ring holds three TQ3 page-heads back to back
// (kTq3Unit bytes each) or two FP8 halves (kSlot each).  The 16-row instance
// keeps two slots of kSlot per wave (kRing) and a second fragment set.  At the
// end of an item the ring is reused for the merge of the 12 wave states.
template <int D>
struct Geo {
  static constexpr int NG = D / 32;                 // 32-channel MFMA k-chunks (TQ3: scale groups)
  static constexpr int NT = D / 16;                 // 16-channel output tiles of P V
  static constexpr int kRows = D / 64;              // 1 KB rows of a staging slot
  static constexpr int kSlot = kRows * 1024;
  static constexpr int kRing = kWaves * 2 * kSlot;
  static constexpr int kTq3Unit = 14 * D;           // one TQ3 page-head
  static constexpr int kWaveRing3 = 3 * kTq3Unit > 2 * kSlot ? 3 * kTq3Unit : 2 * kSlot;
  static constexpr int kRing3 = kWaves * kWaveRing3;
  static constexpr int kSq = NG * 64 * 16;
  static constexpr int kRowMax = kWaves * 16 * 4 + 64; // per-wave query-row maxima (prologue), then the
                                                        // waves' pages left (page loops)
  static constexpr int kKsum = NG * 16 * 4;         // TQ3 offset sums per group and column (prologue)
  static constexpr int kLds = kRing3 + kSq + kRowMax + kKsum;
};

// Staging unit: the bytes a wave moves to one LDS slot.  For TQ3 a unit is
// one page-head (14 d bytes: codes and scales of one KV head); for FP8 a
// page-head (32 d bytes) is two units, its K half and its V half.  Both fit a
// slot of d / 64 rows of 1 KB.  The copy goes straight from HBM to LDS
// (global_load_lds_dwordx4, non-temporal: lane l's 16 bytes of row i land at
// slot + 1024 i + 16 l), so the unit in flight holds no registers.  In a
// partial last row the lanes past the end re-read an in-range address and
// fill the slot's padding, so every load is issued unconditionally and the
// wave's count of outstanding loads is static.
template <int D, bool kMaskTail = false>
__device__ inline void stage_issue(const uint8_t* __restrict__ src, uint8_t* slot, int lane, int bytes) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)slot));
  // 16 * lane, recomputed at every call: kept out of loop-invariant code
  // motion, which would hold one offset register per row across the page loop
  uint32_t l16;
  asm volatile("v_lshlrev_b32 %0, 4, %1" : "=v"(l16) : "v"(lane));
#pragma unroll
  for (int i = 0; i < Geo<D>::kRows; ++i) {
    uint32_t off = 1024 * i + l16;
    // the (wave-uniform) unit address in an SGPR pair, the lane's 32-bit
    // offset in a VGPR; M0 holds the LDS row base.  M0 is an input operand
    // of the asm, so the compiler writes it (and knows it is written); the
    // s_nop gives the one wait state an LDS-DMA load needs after an M0 write
    if (kMaskTail && 1024 * (i + 1) > bytes) {
      // slots packed back to back: the lanes past the end stay inactive (the
      // load is still one instruction, so the count of loads is unchanged)
      if (off < (uint32_t)bytes)
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                     :: "v"(off), "s"(src), "{m0}"(lds + 1024 * i) : "memory");
      continue;
    }
    if (1024 * (i + 1) > bytes && off >= (uint32_t)bytes) off -= 1024 - (bytes & 1023);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(off), "s"(src), "{m0}"(lds + 1024 * i) : "memory");
  }
}

// One row of `bytes` (a multiple of 16, at most 1 KB) copied HBM -> LDS by
// LDS-DMA: lane l moves bytes [16 l, 16 l + 16); lanes past the end are inactive.
__device__ inline void stage_row(const void* __restrict__ src, void* dst, int lane, int bytes) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)dst));
  uint32_t l16;
  asm volatile("v_lshlrev_b32 %0, 4, %1" : "=v"(l16) : "v"(lane));
  if (l16 < (uint32_t)bytes)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(l16), "s"(src), "{m0}"(lds) : "memory");
}

// Issue priority of the wave from its progress through the page loop: the
// SIMD issues from the oldest wave first, so of the three waves of a workgroup
// that share a SIMD (waves w, w + 4, w + 8) the oldest would run ahead and the
// youngest would finish last, alone on its SIMD.  Each wave publishes the
// pages it has left (left[], LDS) and, against its two siblings, takes the
// highest priority when it has the most left and the lowest when it has the
// fewest, so the three finish together.
// left[] is read through a plain LDS pointer: the page loops' asm statements
// clobber memory, so it is read again on every page (a volatile generic
// pointer would compile to flat loads, which count against the vector-memory
// counter the staging waits rely on).
__device__ inline void progress_prio(int* left, int wave, int pages_left) {
  if (__builtin_amdgcn_mbcnt_lo(~0u, 0) == 0) left[wave] = pages_left;
  const int a = __builtin_amdgcn_readfirstlane(left[wave < 8 ? wave + 4 : wave - 8]);
  const int b = __builtin_amdgcn_readfirstlane(left[wave < 4 ? wave + 8 : wave - 4]);
  const int behind = (a < pages_left) + (b < pages_left);     // siblings with fewer pages left
  const int ahead = (a > pages_left) + (b > pages_left);
  if (behind == 2) __builtin_amdgcn_s_setprio(3);
  else if (ahead == 2) __builtin_amdgcn_s_setprio(0);
  else if (behind == 1) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(1);
}

// Wait until at most N vector-memory instructions of this wave are in flight.
// The staging loads are opaque to the compiler (its own conservative wait on
// any LDS-DMA before any LDS read would drain the pipeline), so the waits on
// staged units are placed by hand; the memory clobber keeps the LDS reads of a
// slot after the wait for its unit.
template <int N>
__device__ inline void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// LDS layout of the 4 wave states at the end of an item: channel c = n (D/16)
// + T of query row i of wave w.  Slices of D/16 channels are padded by one
// float and rows by 8, so the 32 lanes that store one (T, r) at a time (16
// slices x 2 rows) hit distinct banks, and reads along c stay conflict-free.
// The wave maxima and denominators follow the states.
template <int D>
struct MergeLayout {
  static constexpr int kSlice = D / 16 + 1;
  static constexpr int kRow = 16 * kSlice + 8;
  static constexpr int kWave = kMaxG * kRow;
  static constexpr int kStates = kWaves * kWave;                 // floats
  // the states, then per-wave maxima and denominators of NR rows and their max
  static constexpr int bytes(int NR) { return (kStates + (2 * kWaves + 1) * NR) * 4; }
  __device__ static inline int at(int w, int i, int n, int T) { return w * kWave + i * kRow + n * kSlice + T; }
};
// 8-row blocks: each wave leaves its state in its own staging ring as soon as
// its page loop ends (no wave waits for another to write): O minus 4 W (the
// TQ3 offset) of its 8 rows, unscaled, at o(i, n, T) (channel n D/16 + T),
// then its running maxima and denominators.
template <int D>
struct OwnLayout {
  static constexpr int kSlice = D / 16 + 1;
  static constexpr int kRow = 16 * kSlice + (D == 256 ? 8 : 0);
  static constexpr int kO = kMaxG * kRow;
  static constexpr int kM = kO, kL = kO + kMaxG;         // maxima, denominators
  static constexpr int kFloats = kO + 2 * kMaxG;
  static constexpr int kStride = Geo<D>::kWaveRing3 / 4;  // floats between the waves' regions
  __device__ static inline int o(int i, int n, int T) { return i * kRow + n * kSlice + T; }
};
static_assert(OwnLayout<256>::kFloats <= OwnLayout<256>::kStride && OwnLayout<128>::kFloats <= OwnLayout<128>::kStride,
              "a wave's state fits its staging ring");
template <int D>
constexpr int kOwnBytes = kWaves * Geo<D>::kWaveRing3 + kWaves * kMaxG * 4;   // the regions, then weights
template <int D>
constexpr int kRotBytes = kOwnBytes<D> + kMaxG * D * 4;   // then rows for the back-rotation
template <int D>
constexpr int kSmemBytes = Geo<D>::kLds > kRotBytes<D> ? Geo<D>::kLds : kRotBytes<D>;

// 16-row blocks keep fp16(q) and its remainder as two fragment sets (2 kSq).
template <int D>
constexpr int kLds16 = Geo<D>::kRing + 2 * Geo<D>::kSq + Geo<D>::kRowMax + Geo<D>::kKsum;
template <int D>
constexpr int kSmemBytes16 = kLds16<D> > MergeLayout<D>::bytes(16) ? kLds16<D> : MergeLayout<D>::bytes(16);
// rotated 16-row instances: the merge layout, then [16][D] rows for the back-rotation
template <int D>
constexpr int kRotBytes16 = MergeLayout<D>::bytes(16) + 16 * D * 4;
template <int D>
constexpr int kSmemRot16 = kSmemBytes16<D> > kRotBytes16<D> ? kSmemBytes16<D> : kRotBytes16<D>;
static_assert(kSmemBytes<256> <= 160 * 1024 && kSmemRot16<256> <= 160 * 1024, "LDS of one workgroup");

template <typename T>
__device__ inline T lds_load(const uint8_t* p) { return *reinterpret_cast<const T*>(p); }

__device__ inline h2 pkrtz(float a, float b) { return __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(a, b)); }

// Four fp32 values -> the fp16 operand of this lane's MFMA row: rows 0..7
// (lo_sel = 0) take hi = fp16(x) (round toward zero), rows 8..15 (lo_sel = -1)
// the remainder fp16(x - hi); hi + lo = x to ~20 bits.
__device__ inline h4 split_rows(const float (&x)[4], float lo_sel) {
  const h2 h01 = pkrtz(x[0], x[1]), h23 = pkrtz(x[2], x[3]);
  const float y0 = fmaf((float)h01[0], lo_sel, x[0]);
  const float y1 = fmaf((float)h01[1], lo_sel, x[1]);
  const float y2 = fmaf((float)h23[0], lo_sel, x[2]);
  const float y3 = fmaf((float)h23[1], lo_sel, x[3]);
  const h2 r01 = pkrtz(y0, y1), r23 = pkrtz(y2, y3);
  return __builtin_shufflevector(r01, r23, 0, 1, 2, 3);
}

// Per-wave running state of the online softmax: O (16 query rows x d
// channels, C layout of the P V MFMAs), W (TQ3: sum of P s per query row and
// the V scale group of the lane's column, same layout), the running max and
// denominator of the query-row column n this lane holds in the score layout.
template <int D>
struct WaveState {
  f4 O[Geo<D>::NT];
  f4 W;
  float m_run, l_run;

  __device__ inline void init() {
#pragma unroll
    for (int T = 0; T < Geo<D>::NT; ++T) O[T] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    W = f4{0.0f, 0.0f, 0.0f, 0.0f};
    m_run = -INFINITY;
    l_run = 0.0f;
  }

  // Online-softmax update for a page's scores s (tokens 4j..4j+3 of query-row
  // column n, hi and lo query rows not yet added; times sc they are in log2
  // units: sc undoes the power-of-two row scaling of the query fragments and,
  // for FP8 pages, applies the layer's k_scale); returns the A
  // operand of P V: rows 0..7 fp16(p), rows 8..15 the remainder.  On a wave's
  // first page (wave-uniform `first`) O and l are still zero: the max is
  // taken as is and nothing is rescaled.
  //
  // MQ (several query tokens per request, causal): token slot k of the page
  // lies dist0 - k tokens before the request's last token, and the lane's
  // query row may see it only if that distance is at least `lim` (dist0 =
  // kNoMask: the page is wholly visible).  A row may then see nothing of a
  // page, even a wave's first, so a running max of -inf is taken as 0 in the
  // exponent.
  //
  // RB = 16 (16 real query rows, q's remainder already summed by a second
  // MFMA): no row pairing, and P comes back as fp16(p) with its remainder in
  // *p_lo, for two P V MFMAs.
  template <bool MQ, int RB = 8>
  __device__ inline h4 softmax(f4 s, float sc, int ntok, float lo_sel, int j, bool first, int dist0 = 0,
                               int lim = 0, h4* p_lo = nullptr) {
    // scores stay in fragment units (score = s sc, sc a power of two, so the
    // product is exact and the exponent below takes it in one fma)
    if (RB == 8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = s[r] + dpp_ror8(s[r]);   // hi + lo query rows
    }
    if (MQ) {
      if (dist0 < kNoMask) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (dist0 - (4 * j + r) < lim) s[r] = -INFINITY;
      }
    } else if (ntok < kPage) {                  // a request's last page: mask its tail
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * j + r >= ntok) s[r] = -INFINITY;
    }
    // the lane's own maximum decides whether any row must move its running
    // max (a row's max exceeds m_run + kRescale iff one of its lanes' does);
    // the row maximum itself, over the four lanes of the column, is needed
    // only on a wave's first page and when some row moves
    const float lm = max4(s[0], s[1], s[2], s[3]) * sc;
    const float pm = (first || __any(lm > m_run + kRescale)) ? max_xor32(max_xor16(lm)) : lm;
    const bool need = pm > m_run + kRescale;
    if (first) {
      m_run = pm;
    } else if (__any(need)) {
      const float m_new = need ? pm : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first page (m_run = -inf)
      l_run *= alpha;
      m_run = m_new;
      // O rows 4j + r belong to query-row columns 4j + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * j + r);
#pragma unroll
        for (int T = 0; T < Geo<D>::NT; ++T) O[T][r] *= ar;
        W[r] *= ar;
      }
    }
    const float m_use = (MQ && m_run == -INFINITY) ? 0.0f : m_run;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sc, -m_use));   // v_exp_f32; 0 for masked tokens
      l_run += p[r];
    }
    if (RB == 16) {
      *p_lo = split_rows(p, -1.0f);
      return split_rows(p, 0.0f);
    }
    return split_rows(p, lo_sel);
  }
};

// Query rows of a work item.  Single-query decode: the G heads of the KV
// head (r0 = 0, rows = R = G, T = 1).  Multi-query: row r = t G + g of the
// request's R = T G rows (query token t, head g), the block holding rows
// r0 .. r0 + rows - 1; query token t is the request's position
// seq_len - T + t and sees the tokens at most that far.
struct RowBlock {
  int T, r0, rows, R;
  int tail_e;    // page of the chunk that is the request's last logical page (-1: none)
  int prev_e;    // page of the chunk that is the request's logical page n - 2 (-1: none)
  int req_last;  // tokens on the request's last page
};

// The TQ3 offset operand (kneg) is built 2^17 above the query units of the
// fragments, so its fp16 parts keep about 22 bits whatever the group sums
// (|x| < 2^-9 in those units puts 4 times a group sum below 2^15).
constexpr float kKnegUp = 131072.0f, kKnegDown = 1.0f / 131072.0f;

// Scores of one TQ3 page-head staged at pg: one 16x16x32 MFMA per 32-channel
// scale group on the codes u (masked windows of the code stream, fp16
// subnormals u 2^(shift - 24), against fragments that carry 2^(24 - shift)),
// its result scaled by the group's fp16 scale of each token.  The offset -4 s(t, g) sum_{c in g} q(c), summed over the
// groups, is one 16x16x16 MFMA that seeds the scores: A = the token scales
// (token n = lane & 15, k = 4 j + e -> group (4 j + e) % NG), B = kneg (the
// lane's query row, minus four times the group sums of q as fp16 hi / lo
// parts, built once per item; the power of two keeps both parts exact).
template <int D, int RB = 8>
__device__ inline f4 tq3_scores(const uint8_t* pg, const h8* sq, int lane, int j, h4 kneg) {
  constexpr int NG = Geo<D>::NG, GB = 3 * NG;       // bytes of a lane's code chunk
  const int n = lane & 15;
  const uint8_t* kp = pg + (4 * n + j) * GB;
  const uint8_t* sp = pg + 12 * D + 8 * ((n >> 2) * NG + (4 * j) % NG) + 2 * (n & 3);
  h4 as;
#pragma unroll
  for (int e = 0; e < 4; ++e) as[e] = lds_load<_Float16>(sp + 8 * e);
  f4 s = __builtin_amdgcn_mfma_f32_16x16x16f16(as, kneg, f4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
  s *= kKnegDown;                                       // kneg carries 2^17 (fp16 range of its parts)
  auto k_scales = [&](int g) { return lds_load<u2>(pg + 12 * D + 8 * (j * NG + g)); };  // tokens 4j..4j+3
  h8 bq = sq[lane];
  h8 bl = RB == 16 ? sq[NG * 64 + lane] : bq;
  u2 sk = k_scales(0);
  f4 sgp = f4{0.0f, 0.0f, 0.0f, 0.0f};                  // the previous group's result and scales:
  u2 skp = u2{0u, 0u};                                  // scaled while the next group's MFMA runs
  auto scale_into = [&](const f4& sg, const u2& sc) {
    const h2 s01 = u2h(sc[0]), s23 = u2h(sc[1]);
    s[0] = fmaf(sg[0], (float)s01[0], s[0]);
    s[1] = fmaf(sg[1], (float)s01[1], s[1]);
    s[2] = fmaf(sg[2], (float)s23[0], s[2]);
    s[3] = fmaf(sg[3], (float)s23[1], s[3]);
  };
#pragma unroll
  for (int b = 0; b < NG / 4; ++b) {
    // the block's 3 code words are read only now, so one block's codes are live at a time
    const uint32_t w0 = lds_load<uint32_t>(kp + 12 * b), w1 = lds_load<uint32_t>(kp + 12 * b + 4),
                   w2 = lds_load<uint32_t>(kp + 12 * b + 8);
    uint32_t x[8];
    code_windows(w0, w1, w2, x);
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const int g = 4 * b + gg;
      // group g: the lane's 8 channels as fp16 subnormals u 2^(shift - 24),
      // in tq3_channel order (the B fragments carry the matching 2^(24 - shift))
      const int w = 4 * (gg & 1);
      const uint32_t m = gg < 2 ? kLoCodes : kHiCodes;
      const h8 a = __builtin_bit_cast(h8, u4{x[w] & m, x[w + 1] & m, x[w + 2] & m, x[w + 3] & m});
      f4 sg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq, f4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
      if (RB == 16) sg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl, sg, 0, 0, 0);
      const u2 sk_g = sk;
      if (g + 1 < NG) {                    // group g + 1's operands load while the MFMA runs
        bq = sq[(g + 1) * 64 + lane];
        if (RB == 16) bl = sq[NG * 64 + (g + 1) * 64 + lane];
        sk = k_scales(g + 1);
      }
      if (g > 0) scale_into(sgp, skp);     // group g - 1, while group g's MFMA runs
      sgp = sg;
      skp = sk_g;
      // pins the order: group g - 1 is scaled and only group g + 1's operands
      // are loaded before group g + 1's MFMA (instruction selection would
      // otherwise sink every scaling below all the MFMAs and keep all their
      // results live)
      if (RB == 16)
        asm volatile("" : "+v"(s), "+v"(bq), "+v"(bl), "+v"(sk), "+v"(sgp), "+v"(skp) :: "memory");
      else
        asm volatile("" : "+v"(s), "+v"(bq), "+v"(sk), "+v"(sgp), "+v"(skp) :: "memory");
    }
  }
  scale_into(sgp, skp);
  return s;
}

// P V of one TQ3 page-head: V = u s as an exact fp16 pair hi + lo; one
// 16x16x32 MFMA per 16-channel tile takes both, its k index running over
// (token 4j + (e & 3), part e >> 2) with P repeated for the two parts.  The
// lane's column keeps one V scale group in every tile, so W += P s (one
// 16x16x16 MFMA, B = the group's scales of tokens 4j..4j+3) holds what the -4
// offset takes off each of its tiles.  vw: the lane's V code words, block b
// in vw[b]; svv: the lane's V scales (its column's group, tokens 4j..4j+3);
// both read from the staged page by the caller, ahead of the scores.
// vdn = 2^-E (the layer's V shift, tq3_v_exponent): the scales enter as s 2^-E
// (exact), so u s 2^-E stays finite in fp16; the epilogue multiplies by 2^E.
template <int D, int RB = 8>
__device__ inline void tq3_pv(h4 pa, f4 (&O)[Geo<D>::NT], f4& W, int lane, int j,
                              const uint32_t (&vw)[Geo<D>::NG / 4][3], u2 svv, h2 vdn, h4 pl = h4{}) {
  constexpr int NG = Geo<D>::NG;
  const h8 pa2 = __builtin_shufflevector(pa, pa, 0, 1, 2, 3, 0, 1, 2, 3);
  const h8 pl2 = __builtin_shufflevector(pl, pl, 0, 1, 2, 3, 0, 1, 2, 3);   // RB 16: P's remainder
  const h2 sv01 = u2h(svv[0]) * vdn, sv23 = u2h(svv[1]) * vdn;
  const h4 sv4 = __builtin_shufflevector(sv01, sv23, 0, 1, 2, 3);
  W = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, sv4, W, 0, 0, 0);
  if (RB == 16) W = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, sv4, W, 0, 0, 0);
#pragma unroll
  for (int b = 0; b < NG / 4; ++b) {
    const u16v u = __builtin_bit_cast(u16v, decode32(vw[b][0], vw[b][1], vw[b][2]));
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int pp = 4 * b + q4;
      // field r of the triple holds (channel a, token 4j + r) low, (b, 4j + r) high
      const h2 a01 = u2h(u[2 * q4]), a23 = u2h(u[2 * q4 + 1]);
      const h2 b01 = u2h(u[8 + 2 * q4]), b23 = u2h(u[9 + 2 * q4]);
      const h2 ha01 = a01 * sv01, ha23 = a23 * sv23, hb01 = b01 * sv01, hb23 = b23 * sv23;
      const h2 la01 = __builtin_elementwise_fma(a01, sv01, -ha01);
      const h2 la23 = __builtin_elementwise_fma(a23, sv23, -ha23);
      const h2 lb01 = __builtin_elementwise_fma(b01, sv01, -hb01);
      const h2 lb23 = __builtin_elementwise_fma(b23, sv23, -hb23);
      const h8 b0 = __builtin_bit_cast(h8, u4{h2u(ha01), h2u(ha23), h2u(la01), h2u(la23)});
      const h8 b1 = __builtin_bit_cast(h8, u4{h2u(hb01), h2u(hb23), h2u(lb01), h2u(lb23)});
      O[2 * pp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa2, b0, O[2 * pp], 0, 0, 0);
      O[2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa2, b1, O[2 * pp + 1], 0, 0, 0);
      if (RB == 16) {
        O[2 * pp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl2, b0, O[2 * pp], 0, 0, 0);
        O[2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl2, b1, O[2 * pp + 1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Scores of one FP8 K half staged at pg (16 tokens x d channels, E4M3):
// codes convert exactly to fp16; lane (n, j) takes channels j d/4 + 8 g + e.
template <int D, int RB = 8>
__device__ inline f4 fp8_scores(const uint8_t* pg, const h8* sq, int lane, int j) {
  const uint8_t* kp = pg + (lane & 15) * D + j * (D / 4);
  f4 s = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int g = 0; g < Geo<D>::NG; ++g) {
    const u2 w = lds_load<u2>(kp + 8 * g);
    const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, false);
    const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, true);
    const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, false);
    const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, true);
    const h8 a = __builtin_bit_cast(h8, u4{h2u(p0), h2u(p1), h2u(p2), h2u(p3)});
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, sq[g * 64 + lane], s, 0, 0, 0);
    if (RB == 16) s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, sq[Geo<D>::NG * 64 + g * 64 + lane], s, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s;
}

// P V of one FP8 V half staged at pg: B = 16 tokens x 16 channels per tile
// (FP8 values are exact in fp16); lane (n, j) holds tokens 4j..4j+3 of
// channels n d/16 + T.
template <int D, int RB = 8>
__device__ inline void fp8_pv(const uint8_t* pg, h4 pa, f4 (&O)[Geo<D>::NT], int lane, int j, h4 pl = h4{}) {
  constexpr int VW = D / 64;                 // dwords of one token row of the lane's channels
  const uint8_t* vp = pg + (4 * j) * D + (lane & 15) * (D / 16);
#pragma unroll
  for (int wi = 0; wi < VW; ++wi) {
    const uint32_t r0 = lds_load<uint32_t>(vp + 4 * wi);
    const uint32_t r1 = lds_load<uint32_t>(vp + D + 4 * wi);
    const uint32_t r2 = lds_load<uint32_t>(vp + 2 * D + 4 * wi);
    const uint32_t r3 = lds_load<uint32_t>(vp + 3 * D + 4 * wi);
#pragma unroll
    for (int bo = 0; bo < 4; bo += 2) {
      const int T = 4 * wi + bo;
      const uint32_t sel = bo | ((4 + bo) << 8) | ((bo + 1) << 16) | ((5 + bo) << 24);
      const uint32_t w01 = __builtin_amdgcn_perm(r1, r0, sel);
      const uint32_t w23 = __builtin_amdgcn_perm(r3, r2, sel);
      const h2 a01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w01, 1.0f, false);   // channel T, tokens 0,1
      const h2 b01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w01, 1.0f, true);    // channel T+1
      const h2 a23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w23, 1.0f, false);
      const h2 b23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w23, 1.0f, true);
      const h4 va = __builtin_bit_cast(h4, u2{h2u(a01), h2u(a23)});
      const h4 vb = __builtin_bit_cast(h4, u2{h2u(b01), h2u(b23)});
      O[T] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, va, O[T], 0, 0, 0);
      O[T + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, O[T + 1], 0, 0, 0);
      if (RB == 16) {
        O[T] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, va, O[T], 0, 0, 0);
        O[T + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vb, O[T + 1], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace

enum AttendMode { kFp8Only = 0, kTq3Only = 1, kBoth = 2 };

// One work item: the partial state of (layer, chunk, KV head) over the pages
// of one format, written to the workspace.  TQ3 is a template parameter so
// each format's code path gets its own register allocation, and each loop
// body is straight-line code (no per-unit branch for the allocator to split
// the accumulators at).
template <int D, bool tq3, bool MQ, int RB = 8, bool ROT = false>
__device__ __forceinline__ void run_item(
    const LayerTable& lt, int hkv, int G, const float* __restrict__ q, const float* __restrict__ q_t, size_t q_ls,
    float qscale, const Plan& plan, int layer, int h, int b, int start, int count, int last_tok, int pidx, int first_id,
    bool holds_tail, uint8_t* smem, const AppendIn* ap, const RowBlock& rb) {
  using GD = Geo<D>;
  constexpr int NG = GD::NG, kSlot = GD::kSlot, kRows = GD::kRows;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, j = lane >> 4;   // C/B column (query row or channel slice), row group
  const float lo_sel = n < 8 ? 0.0f : -1.0f;  // MFMA rows 8..15 carry the fp16 remainders
  const int hq = hkv * G;
  constexpr int NS = RB == 8 ? 3 : 2;        // TQ3 staging slots of a wave
  constexpr int kTs = NS == 3 ? GD::kTq3Unit : kSlot;
  uint8_t* const slot0 = smem + wave * (NS == 3 ? GD::kWaveRing3 : 2 * kSlot);
  uint8_t* const slot1 = slot0 + kSlot;      // FP8: K halves in slot0, V halves in slot1
  h8* const sq = reinterpret_cast<h8*>(smem + (NS == 3 ? GD::kRing3 : GD::kRing));
  int* const s_left = reinterpret_cast<int*>(
      smem + (NS == 3 ? GD::kRing3 : GD::kRing) + (RB == 16 ? 2 : 1) * GD::kSq + kWaves * 16 * 4);
  // FP8 K codes enter the score MFMAs as they are; the layer's k_scale
  // multiplies the fp32 scores (TQ3 K scales are in the group scales)
  const float ks_layer = tq3 ? 1.0f : lt.k_scale[layer];
  const float vup = tq3 ? lt.tq3_v_up[layer] : lt.v_scale[layer];   // fp32 factor of the wave states
  const _Float16 vdn1 = (_Float16)(1.0f / lt.tq3_v_up[layer]);        // 2^-E, exact in fp16
  const h2 vdn = h2{vdn1, vdn1};
  const cptr_i32 list = (cptr_i32)(tq3 ? plan.list_t : plan.list_f);
  const uint8_t* __restrict__ slab = tq3 ? lt.tq3[layer] : lt.fp8[layer];
  const size_t page_bytes = tq3 ? (size_t)tq3_page_bytes(hkv, D) : (size_t)fp8_page_bytes(hkv, D);
  const uint8_t* __restrict__ head = slab + (tq3 ? (size_t)h * tq3_head_bytes(D) : (size_t)h * 2 * kPage * D);
  const int my_pages = count > wave ? (count - wave + kWaves - 1) / kWaves : 0;
  // page of the chunk that this wave takes k-th (chunk_order: with the
  // request's last page in the chunk, that page comes first, to wave 0)
  auto chunk_page = [&](int k) { return chunk_order(wave + kWaves * k, count, holds_tail); };
  // its id (clamped, so reading one id past the end stays in range)
  auto page_id = [&](int k) { return list[start + chunk_page(k < my_pages ? k : my_pages - 1)]; };
  auto page_src = [&](int id) { return head + (size_t)id * page_bytes; };

  // The step's new token, appended in the same launch: the FP8 chunk that
  // holds a request's last logical page (always FP8: it is Recent) writes
  // head h's K and V rows of the token into it, E4M3 round-to-nearest-even
  // saturating like mkv_append, before anything of that page is staged; the
  // wave that stages the page (wave 0, which takes it first) is the one that
  // writes it, so its own loads come after its stores.
  if (!tq3 && ap && ap->k && holds_tail && wave == 0) {
    uint8_t* page = lt.fp8[layer] + (size_t)list[start + count - 1] * page_bytes;
    const int slot = last_tok - 1;
    const size_t row = layer * ap->ls + ((size_t)b * hkv + h) * D;
    const float ksc = lt.k_scale[layer], vsc = lt.v_scale[layer];
    for (int e4 = lane; e4 < 2 * D / 4; e4 += 64) {
      const int kv = e4 >= D / 4, c = 4 * (e4 - kv * (D / 4));
      const float4 x = *reinterpret_cast<const float4*>((kv ? ap->v : ap->k) + row + c);
      const float sc = kv ? vsc : ksc;
      const uint32_t w = e4m3_encode(__fdiv_rn(x.x, sc)) | (e4m3_encode(__fdiv_rn(x.y, sc)) << 8) |
                         (e4m3_encode(__fdiv_rn(x.z, sc)) << 16) | (e4m3_encode(__fdiv_rn(x.w, sc)) << 24);
      *reinterpret_cast<uint32_t*>(page + ((h * 2 + kv) * kPage + slot) * D + c) = w;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // stores done before the page is staged
  }

  // The item's query rows go to LDS first (LDS-DMA into the fragment area,
  // which they leave before the fragments are written), then the first unit(s)
  // of each wave: a wave waits for its query rows alone (the copies complete
  // in order), so the fragments are built while the first pages travel.
  const float* const qsrc = (ROT && tq3) ? q_t : q;
  float* const qbuf = reinterpret_cast<float*>(sq);      // [RB][D] fp32 rows
  auto q_row_ptr = [&](int row) {
    if (MQ) {
      const int r = rb.r0 + row, t = r / G;
      return qsrc + layer * q_ls + ((size_t)(b * rb.T + t) * hq + (size_t)h * G + (r - t * G)) * D;
    }
    return qsrc + layer * q_ls + ((size_t)b * hq + (size_t)h * G + row) * D;
  };
  int q_loads = 0;                                          // wave-uniform
  for (int row = wave; row < rb.rows; row += kWaves) {
    stage_row(q_row_ptr(row), qbuf + row * D, lane, D * 4);
    ++q_loads;
  }
  if (my_pages > 0) {
    if (tq3) {
      stage_issue<D, NS == 3>(page_src(first_id), slot0, lane, tq3_head_bytes(D));   // = page_id(0), from the chunk entry
      wait_vmem<kRows>();                                  // the query rows have landed
    } else {
      const uint8_t* p0 = page_src(first_id);
      stage_issue<D>(p0, slot0, lane, kPage * D);
      stage_issue<D>(p0 + kPage * D, slot1, lane, kPage * D);
      wait_vmem<2 * kRows>();
    }
  } else {
    wait_vmem<0>();
  }
  (void)q_loads;
  __syncthreads();                                          // every wave's query rows

  // ---- B operand of the score MFMAs, shared by the waves through LDS:
  //      query rows 0..G-1 carry fp16(y), rows 8..8+G-1 the remainder; with
  //      16-row blocks all 16 columns are rows, fp16(y) in the first fragment
  //      set and the remainder in the second.  x = q qscale 2^F, with F a
  //      power of two per query row that puts the row's largest |x| in
  //      [128, 256) for FP8 items and in [2^-10, 2^-9) for TQ3 items, and
  //      y = x for FP8.  For TQ3, entry k of a fragment is channel
  //      tq3_channel(k) of the lane's quarter (the order in which tq3_scores
  //      extracts the codes) and y = x 2^(24 - tq3_code_shift(g, k)): the codes
  //      enter the MFMA as fp16 subnormals u 2^(shift - 24), so each product
  //      is u x, and y stays below 2^15.  The matrix cores align a dot
  //      product's terms on their operands' exponent fields, and a subnormal
  //      code counts at exponent -14 however small it is, so terms whose code
  //      sits low in its half would lose their low bits.  TQ3 fp16(y) is
  //      therefore x rounded to the uniform grid 2^-20 (an integer below 2^11
  //      times 2^(4 - shift), exact in fp16): every hi term is a multiple of
  //      2^-20, which the alignment keeps whole; the remainder (below 2^-21)
  //      follows in fp16.  FP8 fp16(x) rounds toward zero.  Either pair holds
  //      x to about 22 bits of the row's maximum whatever the size of q (and
  //      of the layer scales).  Scores are multiplied by 2^-F in fp32.
  //      A thread's row is that of its lane's MFMA column (lane & 15), so the
  //      same F scales its fragments and, later, its column of scores.
  static_assert(NG * 64 <= kThreads, "one fragment entry per thread");
  const bool builds = threadIdx.x < NG * 64;  // this thread builds fragment entry threadIdx.x
  const int fe = threadIdx.x;
  const int fg = fe >> 6, fjj = (fe & 63) >> 4;
  float xq[8];
  float lmax = 0.0f;
  const int qrow_i = RB == 16 ? n : (n & 7);  // this thread's query row (MFMA column n)
  {
    const bool use = qrow_i < rb.rows && builds;
    const float* qrow = qbuf + (use ? qrow_i : 0) * D;
    const int c0 = builds ? (tq3 ? 32 * fg + 8 * fjj : fjj * (D / 4) + 8 * fg) : 0;
    const float4 a = *reinterpret_cast<const float4*>(qrow + c0);
    const float4 c = *reinterpret_cast<const float4*>(qrow + c0 + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      xq[k] = (use ? v[tq3 ? tq3_channel(k) : k] : 0.0f) * qscale;
      lmax = fmaxf(lmax, fabsf(xq[k]));
    }
  }
  // the row's maximum: over the lanes of the row in this wave (RB 8: lanes
  // n and n ^ 8 hold the same row), then over the waves through LDS
  if (lane == 0) s_left[wave] = my_pages;     // pages left, read by the page loops' priorities
  if (RB == 8) lmax = fmaxf(lmax, dpp_ror8(lmax));
  lmax = max_xor32(max_xor16(lmax));
  float* const srm = reinterpret_cast<float*>(smem + (NS == 3 ? GD::kRing3 : GD::kRing) + (RB == 16 ? 2 : 1) * GD::kSq);
  float* const ksum = srm + GD::kRowMax / 4;  // TQ3: per group and column, the sum its offset takes
  if (lane < (RB == 16 ? 16 : 8)) srm[wave * 16 + lane] = lmax;
  __syncthreads();
  float rmax = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) rmax = fmaxf(rmax, srm[w * 16 + qrow_i]);
  int F = rmax > 0.0f ? (tq3 ? -9 : 8) - __builtin_amdgcn_frexp_expf(rmax) : 0;
  F = F < -100 ? -100 : (F > 100 ? 100 : F);
  const float qsc = __builtin_amdgcn_ldexpf(1.0f, -F);   // score factor of this lane's column
  if (builds) {
    const bool hi_codes = (fg & 3) >= 2;      // groups 4b + 2, 4b + 3 take the blocks' high codes
    h8 f0, f1;
    if (tq3) {
      h8 hi, lo;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float x = __builtin_amdgcn_ldexpf(xq[k], F);
        const float hx = __builtin_rintf(__builtin_amdgcn_ldexpf(x, 20));   // |hx| <= 2^11
        const int sh = tq3_code_shift(hi_codes, k);
        hi[k] = (_Float16)__builtin_amdgcn_ldexpf(hx, 4 - sh);             // exact
        lo[k] = (_Float16)__builtin_amdgcn_ldexpf(x - __builtin_amdgcn_ldexpf(hx, -20), 24 - sh);
      }
      if (RB == 16) {
        f0 = hi;
        f1 = lo;
        sq[fe] = f0;
        sq[NG * 64 + fe] = f1;
      } else {
        f0 = lo_sel < 0.0f ? lo : hi;
        f1 = h8{};
        sq[fe] = f0;
      }
    } else if (RB == 16) {
      float x0[4], x1[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x0[k] = __builtin_amdgcn_ldexpf(xq[k], F);
        x1[k] = __builtin_amdgcn_ldexpf(xq[k + 4], F);
      }
      f0 = __builtin_shufflevector(split_rows(x0, 0.0f), split_rows(x1, 0.0f), 0, 1, 2, 3, 4, 5, 6, 7);
      f1 = __builtin_shufflevector(split_rows(x0, -1.0f), split_rows(x1, -1.0f), 0, 1, 2, 3, 4, 5, 6, 7);
      sq[fe] = f0;
      sq[NG * 64 + fe] = f1;
    } else {
      float x0[4], x1[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x0[k] = __builtin_amdgcn_ldexpf(xq[k], F);
        x1[k] = __builtin_amdgcn_ldexpf(xq[k + 4], F);
      }
      f0 = __builtin_shufflevector(split_rows(x0, lo_sel), split_rows(x1, lo_sel), 0, 1, 2, 3, 4, 5, 6, 7);
      f1 = h8{};
      sq[fe] = f0;
    }
    if (tq3) {
      // the column's share of the offset: its fragment values taken back to
      // x units (exact: fp16 times a power of two), summed over the quarter
      // lanes of the group in this wave
      float t = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float back = __builtin_amdgcn_ldexpf(1.0f, tq3_code_shift(hi_codes, k) - 24);
        t = fmaf((float)f0[k] + (RB == 16 ? (float)f1[k] : 0.0f), back, t);
      }
      t = sum_xor32(sum_xor16(t));
      if (lane < 16) ksum[fg * 16 + lane] = t;
    }
  }
  __syncthreads();
  if (kItemTrace && wave0()) trace_time(1);

  // TQ3: B operand of the offset MFMA.  Lane (n, j), k = 4 j + e: minus four
  // times column n's sum over group (4 j + e) % NG, fp16 hi for k < NG, the
  // remainder for NG <= k < 2 NG, 0 beyond.
  h4 kneg = h4{};
  if (tq3) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 4 * j + e;
      const float x = -4.0f * kKnegUp * ksum[(k % NG) * 16 + n];   // the -4 code offset, times the group sum
      const _Float16 hi = (_Float16)x;
      const _Float16 lo = (_Float16)(x - (float)hi);
      kneg[e] = k < NG ? hi : (k < 2 * NG ? lo : (_Float16)0.0f);
    }
  }

  // three slots: page 1 goes out once the query fragments are built (its id,
  // a scalar load, has landed by then)
  if (tq3 && NS == 3 && my_pages > 1)
    stage_issue<D, true>(page_src(page_id(1)), slot0 + kTs, lane, tq3_head_bytes(D));

  WaveState<D> st;
  st.init();
  // MQ: the lane's query row may see tokens at least `lim` before the end
  int lim = 0;
  if (MQ) {
    const int row = RB == 16 ? n : (n & 7);
    lim = row < rb.rows ? rb.T - 1 - (rb.r0 + row) / G : 0;
  }
  auto dist0_of = [&](int e) {
    return e == rb.tail_e ? last_tok - 1 : (e == rb.prev_e ? rb.req_last + kPage - 1 : kNoMask);
  };
  if (tq3) {
    // NS slots: pages k+1 .. k+NS-1 travel while page k is computed; page
    // k+NS-1 goes to the slot page k-1 left
    int id_next = page_id(NS - 1);            // page ids travel one page ahead of their loads
    int s_cur = 0;                            // slot of page k (wave-uniform)
    for (int k = 0; k < my_pages; ++k) {
      progress_prio(s_left, wave, my_pages - k);
      uint8_t* const cur = slot0 + s_cur * kTs;
      if (k + NS - 1 < my_pages) {            // wave-uniform
        const int s_new = s_cur == 0 ? NS - 1 : s_cur - 1;
        const uint8_t* const nsrc = page_src(id_next);
        id_next = page_id(k + NS);
        stage_issue<D, NS == 3>(nsrc, slot0 + s_new * kTs, lane, tq3_head_bytes(D));
        wait_vmem<(NS - 1) * kRows>();        // page k has landed, the next NS - 1 in flight
      } else if (NS == 3 && k + 1 < my_pages) {
        wait_vmem<kRows>();                   // page k has landed, the last one in flight
      } else {
        wait_vmem<0>();                       // the last page has landed
      }
      s_cur = s_cur + 1 == NS ? 0 : s_cur + 1;
      if (kItemTrace && k == 0) trace_time(4 + wave);
      __builtin_amdgcn_sched_barrier(0);
      const int e = chunk_page(k);            // page of the chunk
      const int ntok = (e == count - 1) ? last_tok : kPage;
      // this lane's V code words (its 3 NG bytes of the V code stream) and the
      // V scales of its column's group: with 8-row blocks they are requested
      // before the scores, so they have landed by the P V step; the 16-row
      // instance has no registers to spare and reads them after the softmax
      uint32_t vw[NG / 4][3];
      u2 svv;
      auto read_v = [&]() {
#pragma unroll
        for (int b = 0; b < NG / 4; ++b)
#pragma unroll
          for (int i = 0; i < 3; ++i) vw[b][i] = lds_load<uint32_t>(cur + 6 * D + lane * 3 * NG + 12 * b + 4 * i);
        svv = lds_load<u2>(cur + 13 * D + 8 * (j * NG + (lane & 15) * D / 512));
      };
      if constexpr (RB == 8) read_v();
      const f4 s = tq3_scores<D, RB>(cur, sq, lane, j, kneg);
      h4 pl;
      const h4 pa = st.template softmax<MQ, RB>(s, qsc, ntok, lo_sel, j, k == 0, MQ ? dist0_of(e) : 0, lim, &pl);
      if constexpr (RB == 16) read_v();
      tq3_pv<D, RB>(pa, st.O, st.W, lane, j, vw, svv, vdn, pl);
    }
  } else {
    const float qsc_k = qsc * ks_layer;
    // slot 0 holds K halves, slot 1 V halves: K of page k+1 travels while V of
    // page k is computed, and V of page k+1 while K of page k+1 is
    int id_next = page_id(1);
    for (int k = 0; k < my_pages; ++k) {
      progress_prio(s_left, wave, my_pages - k);
      wait_vmem<kRows>();                     // K of page k has landed
      if (kItemTrace && k == 0) trace_time(4 + wave);
      __builtin_amdgcn_sched_barrier(0);
      const int e = chunk_page(k);
      const int ntok = (e == count - 1) ? last_tok : kPage;
      const f4 s = fp8_scores<D, RB>(slot0, sq, lane, j);
      h4 pl;
      const h4 pa = st.template softmax<MQ, RB>(s, qsc_k, ntok, lo_sel, j, k == 0, MQ ? dist0_of(e) : 0, lim, &pl);
      const bool more = k + 1 < my_pages;     // wave-uniform
      const uint8_t* pn = page_src(id_next);
      id_next = page_id(k + 2);
      if (more) {
        stage_issue<D>(pn, slot0, lane, kPage * D);
        wait_vmem<kRows>();                   // V of page k has landed, K of page k+1 in flight
      } else {
        wait_vmem<0>();
      }
      __builtin_amdgcn_sched_barrier(0);
      fp8_pv<D, RB>(slot1, pa, st.O, lane, j, pl);
      if (more) stage_issue<D>(pn + kPage * D, slot1, lane, kPage * D);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  if (kItemTrace) trace_time(16 + wave);
  wait_vmem<0>();                               // no staging load may land after this point
  const float vscale = vup;
  // this block's rows from r0 (part_acc_index / part_ml_index layout)
  float* __restrict__ ml = plan.part_ml + part_ml_index(plan.np_cap, hkv, rb.R, layer, h, pidx, rb.r0);
  float* __restrict__ pa_out = plan.part_acc + part_acc_index(plan.np_cap, hkv, D, rb.R, layer, h, pidx, rb.r0, 0);
  const size_t slice_stride = (size_t)plan.np_cap * rb.R * kStateSlice;   // between 32-channel slices
  auto state_at = [&](int i, int c) { return (size_t)(c / kStateSlice) * slice_stride + i * kStateSlice + c % kStateSlice; };
  const float l_tot = sum_xor32(sum_xor16(st.l_run));   // sum over the four token rows of column n
  uint32_t opq = 0;
  // rotated TQ3 (uniform): the summed state rows acc' (rows x D in LDS at
  // rbuf) go back to the cache's channels, acc = signs . (H acc') / (c d),
  // c d = 16, H by the fast transform (stage s pairs channels i and i + 2^s)
  const int8_t* const sgn = (ROT && tq3) ? lt.signs[layer] : nullptr;
  auto rotate_back_store = [&](float* rbuf, int rows) {
    for (int hs = 1; hs < D; hs <<= 1) {
      __syncthreads();
      for (int pp = threadIdx.x; pp < rows * D / 2; pp += kThreads) {
        const int i = pp / (D / 2), r = pp - i * (D / 2);
        float* const rr = rbuf + i * D + (r / hs) * 2 * hs + r % hs;
        const float a = rr[0], b2 = rr[hs];
        rr[0] = a + b2;
        rr[hs] = a - b2;
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < rows * D; idx += kThreads) {
      const int c = idx % D;
      const float v = rbuf[idx] * 0.0625f;       // 1 / (c d) = 1/16 at d = 128 and 256
      pa_out[state_at(idx / D, c)] = sgn[c] < 0 ? -v : v;
    }
  };
  if constexpr (RB == 16) {
  __syncthreads();                              // the staging block becomes the merge buffer
  // an opaque zero offset for the merge-buffer addresses below: it keeps the
  // compiler from computing the address of every wave's state before the page
  // loops (and spilling them) instead of here
  asm volatile("" : "+v"(opq));
  // ---- merge of the wave states: each wave rescales its rows to the common
  //      maximum, then the workgroup sums the states in a fixed order
  constexpr int NR = 16;                                 // rows of the wave states
  float* const so = reinterpret_cast<float*>(smem);
  float* const sm = so + MergeLayout<D>::kStates;        // [kWaves][NR] maxima
  float* const sl = sm + kWaves * NR;                    // [kWaves][NR]
  float* const sM = sl + kWaves * NR;                    // [NR] their max
  if (j == 0 && n < rb.rows) {
    sm[wave * NR + n] = st.m_run;
    sl[wave * NR + n] = l_tot;
  }
  __syncthreads();
  if (threadIdx.x < NR) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm[w * NR + threadIdx.x + opq]);
    sM[threadIdx.x] = M;
  }
  __syncthreads();
    // 16 real rows, lane (n, j) holding rows 4j .. 4j + 3: rows 0..7 (j < 2),
    // then rows 8..15 (j >= 2), through the 8-row LDS layout
    for (int pass = 0; pass < 2 && 8 * pass < rb.rows; ++pass) {
      if ((j >> 1) == pass) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * j + r;
          const float mw = sm[wave * NR + row];
          const float wr = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - sM[row]) * vscale;
          const float cw = tq3 ? -4.0f * st.W[r] * wr : 0.0f;     // TQ3 V's -4 offset
#pragma unroll
          for (int T = 0; T < GD::NT; ++T)
            so[MergeLayout<D>::at(wave, 4 * (j & 1) + r, n, T)] = fmaf(st.O[T][r], wr, cw);
        }
      }
      __syncthreads();
      const int rows_p = rb.rows - 8 * pass < 8 ? rb.rows - 8 * pass : 8;
      float* const rbuf = so + MergeLayout<D>::bytes(16) / 4;   // rotated: [16][D], after the merge layout
      for (int idx = threadIdx.x; idx < rows_p * D; idx += kThreads) {
        const int i = idx / D, c = idx - (idx / D) * D;
        const float* src = so + opq + MergeLayout<D>::at(0, i, c / (D / 16), c % (D / 16));
        float acc = 0.0f;
#pragma unroll 4
        for (int w = 0; w < kWaves; ++w) acc += src[w * MergeLayout<D>::kWave];
        if (ROT && sgn)
          rbuf[(8 * pass + i) * D + c] = acc;
        else
          pa_out[state_at(8 * pass + i, c)] = acc;
      }
      __syncthreads();                                  // the layout is rewritten by the next pass
    }
    if (ROT && sgn) rotate_back_store(so + MergeLayout<D>::bytes(16) / 4, rb.rows);
  if (threadIdx.x < rb.rows) {
    const int i = threadIdx.x + opq;
    const float M = sM[i];
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm[w * NR + i];
      const float lw = sl[w * NR + i] * __builtin_amdgcn_exp2f(mw - M);
      L += (mw == -INFINITY) ? 0.0f : lw;
    }
    ml[2 * i] = M;
    ml[2 * i + 1] = L;
  }
  } else {
  // ---- merge of the wave states (8-row blocks).  Each wave writes its state
  //      into its own staging ring (OwnLayout) right away: O rows 4jj + r,
  //      after the swap below lanes 0..31 (j < 2) hold the rows of tile T and
  //      lanes 32..63 those of tile T + NT/2, combined with their fp16
  //      remainder rows, minus 4 W (TQ3 V's offset, whose lane column keeps
  //      one scale group in every tile); all kMaxG rows are stored (rows >= G
  //      hold values nobody reads).  After one barrier, 96 threads turn the
  //      maxima into per-(wave, row) weights, and after a second the
  //      workgroup sums the states in a fixed order.
  using OL = OwnLayout<D>;
  float* const own = reinterpret_cast<float*>(slot0);
  const int jj = j & 1, thalf = j >> 1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float wc = 0.0f;
    if (tq3) {
      const auto pw = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.W[r]), __float_as_uint(st.W[r]), false,
                                                       false);
      wc = -4.0f * (__uint_as_float(pw[0]) + __uint_as_float(pw[1]));
    }
#pragma unroll
    for (int T = 0; T < GD::NT / 2; ++T) {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.O[T][r]),
                                                       __float_as_uint(st.O[T + GD::NT / 2][r]), false, false);
      const float tot = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
      own[OL::o(4 * jj + r, n, T + thalf * (GD::NT / 2))] = tot + wc;
    }
  }
  if (j == 0 && n < kMaxG) {
    own[OL::kM + n] = st.m_run;
    own[OL::kL + n] = l_tot;
  }
  __syncthreads();                              // every wave's state is in place
  asm volatile("" : "+v"(opq));                 // (as above: addresses computed here)
  float* const so = reinterpret_cast<float*>(smem);
  float* const wgt = so + kWaves * OL::kStride;           // [kWaves][kMaxG] weights
  if (threadIdx.x < kWaves * kMaxG) {
    const int w = threadIdx.x / kMaxG, i = threadIdx.x % kMaxG;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, so[v * OL::kStride + OL::kM + i + opq]);
    const float mw = so[w * OL::kStride + OL::kM + i];
    wgt[w * kMaxG + i] = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M) * vscale;
    if (w == 0 && i < rb.rows) {                // the partial's (m, l)
      float L = 0.0f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float mv = so[v * OL::kStride + OL::kM + i + opq];
        const float lv = so[v * OL::kStride + OL::kL + i] * __builtin_amdgcn_exp2f(mv - M);
        L += (mv == -INFINITY) ? 0.0f : lv;
      }
      ml[2 * i] = M;
      ml[2 * i + 1] = L;
    }
  }
  __syncthreads();
  auto sum_at = [&](int i, int c) {
    const float* src = so + opq + OL::o(i, c / (D / 16), c % (D / 16));
    const float* wi = wgt + opq + i;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc = fmaf(src[w * OL::kStride], wi[w * kMaxG], acc);
    return acc;
  };

  if (ROT && sgn) {                                     // rotated TQ3 (uniform)
    float* const rbuf = so + kOwnBytes<D> / 4;          // [rows][D], after the regions and weights
    for (int idx = threadIdx.x; idx < rb.rows * D; idx += kThreads) {
      const int i = idx / D, c = idx - (idx / D) * D;
      rbuf[idx] = sum_at(i, c);
    }
    rotate_back_store(rbuf, rb.rows);
  } else {
    for (int idx = threadIdx.x; idx < rb.rows * D; idx += kThreads) {
      const int i = idx / D, c = idx - (idx / D) * D;
      pa_out[state_at(i, c)] = sum_at(i, c);   // ordinary stores: the merge, next on the stream, reads them from the caches
    }
  }
  }
  if (kItemTrace && wave0()) {
    trace_time(2);
    trace_mark(3, (uint64_t)count | ((uint64_t)tq3 << 32) | ((uint64_t)h << 40) | ((uint64_t)b << 48));
  }
}


// MODE selects which format's work items the launch takes (kBoth: the FP8
// items first, then the TQ3 items, in one grid so the small FP8 share runs
// alongside the TQ3 stream; each item runs its own format's code path).
// 40 KB of LDS and at most 168 VGPRs per thread: kAttendWgPerCu = 3
// workgroups per CU (the TQ3 page loop needs about 160 registers without
// spills).
// MQ: several query tokens per request (plan.n_query), their rows split in
// plan.nblk blocks, one work item per (chunk, KV head, block); causal masks on
// the request's last two logical pages.
// RB: query rows per item, 8 (MFMA rows 0..7, remainders in 8..15) or, for
// multi-query blocks, 16 (remainders through second MFMAs; 48 KB of LDS).
// ROT: some layer has rotated TQ3 pages: TQ3 items read q_t (the rotated
// queries) and rotate their partial states back.
template <int D, int MODE, bool MQ, int RB, bool ROT = false>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(kAttendWavesPerSimd, kAttendWavesPerSimd))) attend_kernel(
        LayerTable lt, int n_layers, int hkv, int G, const float* __restrict__ q, const float* __restrict__ q_t,
        size_t q_ls, float qscale, Plan plan, AppendIn ap) {
  __shared__ __align__(16) uint8_t smem[RB == 16 ? (ROT ? kSmemRot16<D> : kSmemBytes16<D>) : kSmemBytes<D>];

  static_assert(kWaves == kItemWaves, "a chunk-table entry holds the first page of every wave");
  if (kItemTrace && wave0()) trace_time(0);
  const int nblk = MQ ? plan.nblk : 1;
  // Items: the TQ3 ones first, then the FP8 ones; within a format item
  // ((chunk L + layer) Hkv + h) nblk + blk, so an item's chunk does not depend
  // on the chunk counts and the TQ3 entry of the workgroup's first item is
  // requested together with those counts (clamped into the table; used only if
  // the item turns out to be a TQ3 one).
  // (32-bit unsigned index arithmetic: items per launch stay far below 2^31)
  const unsigned per_chunk = (unsigned)(n_layers * hkv * nblk);
  const cptr_i16 tab_t = (cptr_i16)plan.chunks_t, tab_f = (cptr_i16)plan.chunks_f;
  const int spec = (int)(blockIdx.x / per_chunk);
  const i16v cd_spec = (MODE != kFp8Only && plan.table_cap > 0) ? tab_t[spec < plan.table_cap ? spec : plan.table_cap - 1]
                                                                 : i16v{};
  // a workspace without this batch's plan is refused, not read
  if (plan.totals[T_STAMP] != plan_stamp(plan)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(plan.status, kDevNoPlan);
    return;
  }
  const int ncf = MODE == kTq3Only ? 0 : plan.totals[T_NCF];
  const int nct = MODE == kFp8Only ? 0 : plan.totals[T_NCT];
  const unsigned items_t = per_chunk * nct;
  const unsigned items = per_chunk * ncf + items_t;

  for (unsigned item = blockIdx.x; item < items; item += gridDim.x) {
    const bool tq3 = item < items_t;
    const unsigned it = tq3 ? item : item - items_t;
    const int blk = MQ ? (int)(it % (unsigned)nblk) : 0;
    const unsigned itc = MQ ? it / (unsigned)nblk : it;
    const int h = (int)(itc % (unsigned)hkv);
    const int layer = (int)((itc / (unsigned)hkv) % (unsigned)n_layers);
    const int chunk = (int)(itc / (unsigned)(hkv * n_layers));
    const i16v cd = (tq3 && item == blockIdx.x) ? cd_spec : (tq3 ? tab_t : tab_f)[chunk];
    const int b = cd[0], start = cd[1], count = chunk_pages(cd[2]), last_tok = chunk_last_tok(cd[2]), pidx = cd[3];
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int first_id = cd[4];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) first_id = wv == w ? cd[4 + w] : first_id;
    const bool holds_tail = (cd[2] & kChunkHoldsTail) != 0;
    if (pidx >= plan.np_cap) {               // plan made for fewer layers than this call
      if (threadIdx.x == 0) atomicOr(plan.status, kDevBadSeqLen);
      continue;
    }
    RowBlock rb{1, 0, G, G, -1, -1, 0};
    if (MQ) {
      const cptr_i32 req = (cptr_i32)plan.req;
      const int rowlen = plan.batch + 1;
      const int prev_fmt = req[R_PREVFMT * rowlen + b], prev_idx = req[R_PREVIDX * rowlen + b];
      rb.T = plan.n_query;
      rb.R = rb.T * G;
      rb.r0 = blk * RB;
      rb.rows = rb.R - rb.r0 < RB ? rb.R - rb.r0 : RB;
      rb.tail_e = holds_tail ? count - 1 : -1;
      rb.prev_e = (prev_fmt == (tq3 ? 1 : 0) && prev_idx >= start && prev_idx < start + count) ? prev_idx - start : -1;
      rb.req_last = req[R_TAIL * rowlen + b];
    }
    if (MODE != kFp8Only && tq3)
      run_item<D, true, MQ, RB, ROT>(lt, hkv, G, q, q_t, q_ls, qscale, plan, layer, h, b, start, count, last_tok, pidx, first_id,
                                holds_tail, smem, nullptr, rb);
    if (MODE != kTq3Only && !tq3)
      run_item<D, false, MQ, RB, ROT>(lt, hkv, G, q, q_t, q_ls, qscale, plan, layer, h, b, start, count, last_tok, pidx, first_id,
                                 holds_tail, smem, (holds_tail && (!MQ || plan.n_query == 1)) ? &ap : nullptr, rb);
    __syncthreads();
  }
}

// One workgroup per CU (a workgroup fills its CU's registers), each taking
// work items blockIdx.x, blockIdx.x + gridDim.x, ...: a grid larger than the
// CU count would only add workgroups that wait for a CU to free up.
static int cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static dim3 attend_grid(long cap) {
  const long cus = cu_count();
  return dim3((unsigned)(cap < cus ? (cap > 0 ? cap : 1) : cus));
}

// Queries of rotated TQ3 pages: q' = H (signs . q) / (c d) per row of D
// channels (1 / (c d) = 1/16 at d = 128 and 256), one workgroup of D threads
// per row, the butterflies in LDS; rows of layers without signs are copied.
template <int D>
__global__ void __launch_bounds__(256) rotate_q_kernel(const float* __restrict__ q, float* __restrict__ qr,
                                                      int rows_per_layer, LayerTable lt) {
  __shared__ float buf[D];
  const int row = blockIdx.x, c = threadIdx.x;
  const int8_t* const sg = lt.signs[row / rows_per_layer];
  const float x = q[(size_t)row * D + c];
  if (!sg) {                                         // uniform
    qr[(size_t)row * D + c] = x;
    return;
  }
  buf[c] = sg[c] < 0 ? -x : x;
  for (int hs = 1; hs < D; hs <<= 1) {
    __syncthreads();
    const float a = buf[c & ~hs], b = buf[c | hs];
    __syncthreads();
    buf[c] = (c & hs) ? a - b : a + b;
  }
  __syncthreads();
  qr[(size_t)row * D + c] = buf[c] * 0.0625f;
}

template <int MODE, bool MQ, int RB>
static void launch_attend_t(const Geometry& g, const LayerTable& lt, int n_layers, const float* q,
                            size_t q_ls, float qscale, const Plan& plan, const AppendIn& ap,
                            hipStream_t stream) {
  // rotated TQ3 pages read rotated queries (every query row of the launch:
  // batch x query tokens x heads per layer); FP8-only launches need none
  const float* q_t = q;
  const bool rot = lt.any_signs && MODE != kFp8Only;
  if (rot) {
    const int rows = plan.batch * (MQ ? plan.n_query : 1) * g.hq;
    if (rows > 0) {
      if (g.d == 256)
        hipLaunchKernelGGL(rotate_q_kernel<256>, dim3(n_layers * rows), dim3(256), 0, stream, q, plan.q_rot, rows, lt);
      else
        hipLaunchKernelGGL(rotate_q_kernel<128>, dim3(n_layers * rows), dim3(128), 0, stream, q, plan.q_rot, rows, lt);
    }
    q_t = plan.q_rot;
  }
  // partials per layer bound the items of either format, or of both together
  const dim3 grid = attend_grid((long)n_layers * g.hkv * plan.np_cap * (MQ ? plan.nblk : 1)), block(kThreads);
  if (g.d == 256) {
    if (rot)
      hipLaunchKernelGGL((attend_kernel<256, MODE, MQ, RB, MODE != kFp8Only>), grid, block, 0, stream, lt, n_layers,
                         g.hkv, g.G, q, q_t, q_ls, qscale, plan, ap);
    else
      hipLaunchKernelGGL((attend_kernel<256, MODE, MQ, RB>), grid, block, 0, stream, lt, n_layers, g.hkv, g.G, q,
                         q_t, q_ls, qscale, plan, ap);
  } else {
    if (rot)
      hipLaunchKernelGGL((attend_kernel<128, MODE, MQ, RB, MODE != kFp8Only>), grid, block, 0, stream, lt, n_layers,
                         g.hkv, g.G, q, q_t, q_ls, qscale, plan, ap);
    else
      hipLaunchKernelGGL((attend_kernel<128, MODE, MQ, RB>), grid, block, 0, stream, lt, n_layers, g.hkv, g.G, q,
                         q_t, q_ls, qscale, plan, ap);
  }
}

// Streaming-read probe: units of kProbeUnit bytes (one TQ3 page-head at
// d = 256) copied HBM -> LDS by the page-staging loads (stage_issue: LDS-DMA,
// 16 bytes per lane, non-temporal), three units in flight per wave as in the
// TQ3 page loop, one 12-wave workgroup per CU, nothing computed but an XOR of
// each unit's first word, which lane 0 of each wave leaves in sink.
constexpr int kProbeUnit = 14 * 256;
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const uint8_t* __restrict__ src, unsigned n_units,
                                                               uint32_t* __restrict__ sink) {
  __shared__ __align__(16) uint8_t ring[kWaves * Geo<256>::kWaveRing3];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned gw = blockIdx.x * kWaves + wave, nw = gridDim.x * kWaves;
  const int mine = gw < n_units ? (int)((n_units - 1 - gw) / nw + 1) : 0;   // units gw, gw + nw, ...
  uint8_t* const slot0 = ring + wave * Geo<256>::kWaveRing3;
  auto unit = [&](int k) { return src + (size_t)(gw + (unsigned)k * nw) * kProbeUnit; };
  uint32_t x = 0;
  if (mine > 0) stage_issue<256, true>(unit(0), slot0, lane, kProbeUnit);
  if (mine > 1) stage_issue<256, true>(unit(1), slot0 + kProbeUnit, lane, kProbeUnit);
  int s_cur = 0;
  for (int k = 0; k < mine; ++k) {
    if (k + 2 < mine) {
      stage_issue<256, true>(unit(k + 2), slot0 + (s_cur == 0 ? 2 : s_cur - 1) * kProbeUnit, lane, kProbeUnit);
      wait_vmem<2 * Geo<256>::kRows>();
    } else if (k + 1 < mine) {
      wait_vmem<Geo<256>::kRows>();
    } else {
      wait_vmem<0>();
    }
    x ^= lds_load<uint32_t>(slot0 + s_cur * kProbeUnit);
    s_cur = s_cur == 2 ? 0 : s_cur + 1;
  }
  if (lane == 0) sink[gw] = x;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, hipStream_t stream) {
  const size_t units = bytes / kProbeUnit;
  size_t groups = (size_t)cu_count();
  if (groups > sink_words / kWaves) groups = sink_words / kWaves;
  if (groups < 1) groups = 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)groups), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(src), (unsigned)units, sink);
  return hipGetLastError();
}

size_t stream_read_unit() { return kProbeUnit; }

hipError_t launch_partial_mfma(int which, const Geometry& g, const LayerTable& lt, int n_layers,
                               const float* q, size_t q_layer_stride, float qscale,
                               const Plan& plan, const AppendIn& ap, hipStream_t stream) {
  // 16-row blocks: multi-query with more than 8 rows per KV head, or one
  // query token with 9..16 heads per KV head (then the in-launch append and
  // the format-only launches apply as in the 8-row instance)
  if (plan.rowblk == 16 && which == 0)
    launch_attend_t<kFp8Only, true, 16>(g, lt, n_layers, q, q_layer_stride, qscale, plan, ap, stream);
  else if (plan.rowblk == 16 && which == 1)
    launch_attend_t<kTq3Only, true, 16>(g, lt, n_layers, q, q_layer_stride, qscale, plan, ap, stream);
  else if (plan.rowblk == 16)
    launch_attend_t<kBoth, true, 16>(g, lt, n_layers, q, q_layer_stride, qscale, plan, ap, stream);
  else if (plan.n_query > 1)
    launch_attend_t<kBoth, true, 8>(g, lt, n_layers, q, q_layer_stride, qscale, plan, ap, stream);
  else if (which == 0)
    launch_attend_t<kFp8Only, false, 8>(g, lt, n_layers, q, q_layer_stride, qscale, plan, ap, stream);
  else if (which == 1)
    launch_attend_t<kTq3Only, false, 8>(g, lt, n_layers, q, q_layer_stride, qscale, plan, ap, stream);
  else
    launch_attend_t<kBoth, false, 8>(g, lt, n_layers, q, q_layer_stride, qscale, plan, ap, stream);
  return hipGetLastError();
}

int read_item_trace(uint64_t* host, size_t words) {
  if (!kItemTrace) return -1;
  const size_t n = words < (size_t)kTraceBlocks * kTraceSlots ? words : (size_t)kTraceBlocks * kTraceSlots;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_item_trace), n * sizeof(uint64_t), 0, hipMemcpyDeviceToHost) == hipSuccess
             ? 0
             : -2;
}

}  // namespace mkv
