// HIP kernels for gfx950 (CDNA4): MXFP8 partial amax, amax MAX-combine, E8M0 scales and the
// partial E4M3 cast of a contiguous fragment of a flattened 2-D weight; the cast with the scales
// derived in-kernel from the combined amax; and a single-pass quantize (amax, scales and cast
// from one read) for fragments that own every block they touch.
//
// What is computed follows "Support row-only MXFP8 distributed master-weight casts"
// (TransformerEngine PR 3488, sections Changes and the flow diagram of the Greptile summary)
// with the OCP MX / OFP8 rules for blocks, scales and E4M3; the public contract is in
// include/mxfp8_partial.h.
//
// Design (MI355X first; no matrix cores, since nothing here is a contraction):
//  * A workgroup owns a tile of one 32-row band (the height of a column-wise block) and 64 * E
//    columns, E = elements per 16-byte chunk (8 for BF16, 4 for FP32); each of its four waves
//    takes 8 of the rows.  Each lane streams one 16-byte chunk per row, so every load
//    instruction of a wave covers 1 KiB of contiguous HBM.  Column-wise maxima stay in the
//    lane's registers and meet over the four waves in LDS; row-wise maxima are reduced over the
//    32/E lanes that share a 32-value block with DPP (quad_perm, row_half_mirror), no LDS round
//    trip.  One read of the input feeds both directions.
//  * A wave issues all of a tile's loads before it uses any value (one memory round trip per
//    tile), and large launches hold a measured number of resident workgroups per CU.
//  * amax is handled as unsigned integers on |x|'s bit pattern (exact, independent of the
//    floating-point mode); BF16 pairs use v_pk_max_u16.
//  * The cast scales with v_ldexp_f32 (exact, denormals preserved), saturates with v_med3_f32
//    and converts pairs with v_cvt_pk_fp8_f32 (OCP E4M3, round to nearest even on gfx950).
//  * The column-wise direction and BF16 pre-rounding are compile-time template booleans, so
//    a row-only call carries no column-wise code (the runtime-guard version measured on the
//    pages cost amax 21-35%).
//  * Tiles wholly inside the fragment run branch-free; tiles the fragment boundary cuts take
//    an element-masked path.  The amax entry of a block wholly inside a piece is written by
//    its single owner without being read (no other fragment touches that block); blocks a
//    boundary cuts use an atomic max, so pieces sharing one amax buffer merge correctly in
//    any order.
//  * Workgroup ids are remapped so consecutive tiles (one band's amax entries) land on the
//    same XCD's L2.
//  * Layouts the vector path cannot take (rows that are not whole 16-byte chunks: cols % 8 != 0
//    for BF16, cols % 4 != 0 for FP32) run an element-wise kernel: one lane per column, same
//    band tiling, same results.  Any alignment of input and outputs stays on the vector path
//    (dword loads with a 2-byte realign, window stores).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "mxfp8_internal.h"

namespace mxfp8 {
namespace {

constexpr int kBlockLen = 32;     // MX block length
constexpr int kWaveSize = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWaveSize * kWavesPerGroup;
constexpr int kNumXcd = 8;        // MI355X: 8 XCDs, workgroups dispatched round-robin
// Occupancy of the vector kernels, per kernel and element type, chosen by measurement on
// MI355X.  kAmax / kAmaxSmall / kCast are the resident waves per SIMD the register allocator
// must allow.  Large launches (kSmallLaunchTiles tiles or more) stream best with few resident
// workgroups per CU (kAmaxCap / cast_cap / kQuantCap: more only add contention, fewer starve
// the stream);
// the kernels' register use would let more in, so such a launch reserves enough LDS to hold
// residency at the cap.  Small launches (a single rank's fragment) need every resident
// workgroup they can get to fill the GPU in one round: no cap, and the amax has a variant
// compiled for more waves.
template <typename T>
struct Occupancy {
  static constexpr int kAmax = 4;
  static constexpr int kAmaxSmall = 6;
  static constexpr int kCast = sizeof(T) == 2 ? 3 : 2;
  static constexpr int kAmaxCap = 4;
  static constexpr int kQuantCap = 5;
  // cast: 3 for BF16 with both directions, else 4; cast with fused scales: 5 with both
  // directions, else no cap (0)
  static constexpr int cast_cap(bool col, bool fuse) {
    return fuse ? (col ? 5 : 0) : (sizeof(T) == 2 && col ? 3 : 4);
  }
};
constexpr int64_t kSmallLaunchTiles = 2048;  // below this many tiles: small-launch settings
// Below these many tiles the cast splits its tiles (cast_vec_kernel's kSplit): 4 ways under
// 1024 tiles, 8 ways under 64.  Measured (graph replays): 1024x1024 BF16 quarter 6.74 -> 3.12
// us, 4096x4096 BF16 quarter 9.63 -> 6.38 us; an 8-way split of the 128 tiles of the 1024x1024
// FP32 cast and a 4-way split of 1024 tiles or more ran slower.
constexpr int64_t kSplit4Tiles = 1024;
constexpr int64_t kSplit8Tiles = 64;
// Below this many tiles the amax, whose band must stay in one workgroup (its column-wise
// blocks are 32 rows), takes wider workgroups instead: 8 waves of 4 rows.  Measured (graph
// replays): 1024x1024 BF16 full 3.58 -> 3.38 us, quarter at offset 17 6.52 -> 5.89 us,
// 4096x4096 FP32 quarter 7.06 -> 6.42 us; 16 waves of 2 rows ran 3-12% slower than 8.
constexpr int64_t kAmax8Tiles = 1024;

// The runtime-guard ablation library (built with MXFP8_RUNTIME_GUARDS=1 by build.py
// --ablation) runs the amax and the plain cast of rows of whole chunks through one kernel per
// dtype for row-only and bidirectional calls, the column-wise work selected at run time by a
// test of the column-wise pointer: the kernels the pages measured before the compile-time
// specialization.  The product library (MXFP8_RUNTIME_GUARDS=0) takes those kernels only for
// small calls that hold both directions (one_launch_for_both); everything else runs the
// compile-time specialized kernels.
constexpr bool kRuntimeGuards = MXFP8_RUNTIME_GUARDS != 0;

struct TileArgs {
  int64_t rows, cols, start, end;
  const void* input;
  void* amax_row;
  int64_t ld_ar;
  void* amax_col;
  int64_t ld_ac;
  uint8_t* scale_row;  // read by the cast; written by the fused scales + cast
  int64_t ld_sr;
  uint8_t* scale_col;
  int64_t ld_sc;
  uint8_t* data_row;
  uint8_t* data_col;
  int64_t band0;   // first 32-row band the fragment touches
  int64_t ntc;     // tiles per band
  int64_t ntiles;  // bands * ntc
  int32_t col_vec; // amax_col rows are 16-byte aligned: column entries move as 16-byte vectors
  int32_t row_vec;  // amax_row rows are 16-byte aligned: a tile's row entries move as vectors
  int32_t in_shift2;  // BF16 input with input - start at 2 mod 4 bytes: chunks need a 2-byte shift
  int32_t mo_row, mo_col;  // (data - start) mod 4 of each output: 0 = chunks store directly
  int32_t nt_row, nt_col;  // each output row starts on a 64-byte boundary: streaming stores
  int32_t sc_vec;  // scale_col rows aligned to a chunk's E bytes: a lane's scale bytes are one load
  int32_t shift;   // line-owned cast tiles: flat offset of every tile column (0 elsewhere)
  int32_t row_pair, col_pair;  // BF16 amax rows start on 4-byte boundaries: entries 2k, 2k + 1
                               // share an aligned 32-bit word
  int32_t amax_own;  // no other piece of the launch has this piece's amax arrays: the BF16
                     // merges of cut blocks are a load and a store, not compare-and-swap
  int64_t tile0;   // tiles of the piece that earlier launches of its group covered
};

// One launch covers up to kMaxGroup pieces that share a kernel specialization: tiles are
// numbered piece after piece.  A group with more than kMaxLaunchGroups workgroups goes out as
// several launches, so no grid comes near the 2^32 work-items a dispatch can hold.  first[k]
// is the first tile of piece k counted from the launch's first workgroup: 0 for a piece that
// an earlier launch of the group began (its tile0 then counts the tiles already covered), and
// kNoPiece for one that starts after the launch and for the unused entries (k >= n).  A launch
// holds fewer than 2^31 tiles, so every entry is below 2^31.  The header comes first and is
// 68 bytes, so one scalar load fetches it.
constexpr int kMaxGroup = 16;
constexpr int64_t kMaxLaunchGroups = int64_t(1) << 20;
constexpr uint32_t kNoPiece = 0x7FFFFFFFu;  // beyond every tile of a launch
static_assert(kMaxLaunchGroups * kWavesPerGroup < kNoPiece, "tiles of a launch below kNoPiece");
struct GroupArgs {
  uint32_t first[kMaxGroup];
  int32_t n;
  TileArgs piece[kMaxGroup];
};

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ small device helpers

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kCtrl, 0xF, 0xF, false);
}

// Max over aligned groups of kLanes lanes (4 or 8); every lane of the group gets the result.
template <int kLanes>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  v = umax(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]: lane ^ 1
  v = umax(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (kLanes >= 8) v = umax(v, dpp<0x141>(v));  // row_half_mirror: other quad
  static_assert(kLanes == 4 || kLanes == 8, "group of 4 or 8 lanes");
  return v;
}

// Max over each 32-lane half of the wave (one row-wise block per half in the element path).
__device__ __forceinline__ uint32_t half_wave_max(uint32_t v) {
  v = umax(v, dpp<0xB1>(v));
  v = umax(v, dpp<0x4E>(v));
  v = umax(v, dpp<0x141>(v));
  v = umax(v, dpp<0x140>(v));   // row_mirror: the other 8 lanes of the 16-lane row
  v = umax(v, (uint32_t)__shfl_xor((int)v, 16));
  return v;
}

// FP32 bit pattern rounded to the nearest BF16 value (ties to even), as an FP32 bit pattern.
// Integer arithmetic: exact for normal and subnormal inputs alike.
__device__ __forceinline__ uint32_t round_bf16_bits(uint32_t u) {
  return (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
}

// Dispatch round-robins consecutive workgroup ids over the XCDs; renumber them so that each
// XCD works through one contiguous range of tiles: XCD x takes per + 1 ids if x < rem, else
// per, starting at x * per + min(x, rem).  32-bit and branch-free (a launch holds at most
// kMaxLaunchGroups workgroups).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t wg, uint32_t nwg) {
  const uint32_t per = nwg / kNumXcd, rem = nwg % kNumXcd;
  const uint32_t xcd = wg % kNumXcd, idx = wg / kNumXcd;
  return xcd * per + min(xcd, rem) + idx;
}

// The fields of a piece that a tile's first loads depend on, held in scalar registers at one
// point: the compiler then issues their scalar loads together and waits once.  Left to itself
// it puts each load next to its first use, often behind a branch of its own, and every such
// load is one more round trip before the tile's first global load; in a launch of one round
// all workgroups start cold and wait for each of them.
__device__ __forceinline__ void pin_tile_fields(const GroupArgs& g, int k) {
  const TileArgs& p = g.piece[k];
  asm volatile("" ::"s"(g.first[k]), "s"(p.tile0), "s"(p.rows), "s"(p.cols), "s"(p.start),
               "s"(p.end), "s"(p.input), "s"(p.band0), "s"(p.ntc), "s"(p.ntiles),
               "s"(p.in_shift2), "s"(p.shift));
}

// The same for the cast, plus what its common tile's path test and scale loads read.
__device__ __forceinline__ void pin_cast_fields(const GroupArgs& g, int k) {
  const TileArgs& p = g.piece[k];
  asm volatile("" ::"s"(g.first[k]), "s"(p.tile0), "s"(p.rows), "s"(p.cols), "s"(p.start),
               "s"(p.end), "s"(p.input), "s"(p.band0), "s"(p.ntc), "s"(p.ntiles),
               "s"(p.in_shift2), "s"(p.shift), "s"(p.nt_row), "s"(p.nt_col), "s"(p.sc_vec),
               "s"(p.scale_row), "s"(p.ld_sr), "s"(p.scale_col), "s"(p.ld_sc));
}

// The launch's header and grid size, held in scalar registers at one point (one batch of
// scalar loads, one round trip) ahead of the workgroup's tile and piece.
__device__ __forceinline__ void pin_header(const GroupArgs& g) {
  asm volatile("" ::"s"(gridDim.x), "s"(g.first[1]), "s"(g.first[2]), "s"(g.first[3]),
               "s"(g.first[4]), "s"(g.first[5]), "s"(g.first[6]), "s"(g.first[7]),
               "s"(g.first[8]), "s"(g.first[9]), "s"(g.first[10]), "s"(g.first[11]),
               "s"(g.first[12]), "s"(g.first[13]), "s"(g.first[14]), "s"(g.first[15]));
  static_assert(kMaxGroup == 16, "pin_header names every entry of first[] after the first");
}

// Piece of a grouped launch that tile t of the launch belongs to: the number of later pieces
// whose first tile is at or before t (first[] never decreases, unused entries never match).
// Uniform, and branch-free over all kMaxGroup entries, so the header arrives in one scalar
// load: a loop over the pieces waited for one load per piece before the tile's first global
// load.  Every entry and t are below 2^31, so first[j] - t - 1 is negative exactly when
// first[j] <= t, and its sign bit counts the piece: three scalar instructions per entry (a
// comparison turned into a count went through vector registers, and the extra prologue time
// of every workgroup cost the full-size cast 1%).
__device__ __forceinline__ int piece_of(const GroupArgs& g, uint32_t t) {
  const uint32_t nt = ~t;  // first[j] - t - 1 == first[j] + ~t
  uint32_t k = 0;
#pragma unroll
  for (int j = 1; j < kMaxGroup; ++j) k += (g.first[j] + nt) >> 31;
  return (int)k;
}

// ------------------------------------------------------------------ amax entries

// Global memory at an address computed as an integer (a pointer masked to its dword).  A plain
// pointer made from an integer is a generic one, and generic (flat) accesses count against the
// LDS / scalar-load counter as well, so that every wait for one also waits for the others;
// these are global accesses.
typedef __attribute__((address_space(1))) const uint32_t global_cu32;
typedef __attribute__((address_space(1))) uint32_t global_u32;

__device__ __forceinline__ global_u32* global_dword(uintptr_t a) {
  return reinterpret_cast<global_u32*>(a & ~uintptr_t(3));
}
__device__ __forceinline__ global_cu32* global_cdword(uintptr_t a) {
  return reinterpret_cast<global_cu32*>(a & ~uintptr_t(3));
}

// Compare-and-swap of a global dword; returns the value it found.
__device__ __forceinline__ uint32_t global_cas(global_u32* w, uint32_t expected, uint32_t desired) {
  __hip_atomic_compare_exchange_strong(w, &expected, desired, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return expected;
}

// Atomic max into N amax entries at once; bit i of `active` selects entry i.  Amax values are
// non-negative, so unsigned order on the bit patterns is float order.  FP32 entries use the
// hardware's unsigned atomic max, which returns nothing to wait for.
template <int N>
__device__ __forceinline__ void atomic_max_entries(uint32_t* const (&p)[N],
                                                   const uint32_t (&v)[N], uint32_t active) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    if ((active >> i) & 1u) atomicMax(p[i], v[i]);
}

// BF16 entries have no 16-bit atomic max: each goes through a compare-and-swap on the aligned
// 32-bit word holding it.  All words are read first and all swaps issued together; only swaps
// that lost a race are retried, with the value they observed.
template <int N>
__device__ __forceinline__ void atomic_max_entries(uint16_t* const (&p)[N],
                                                   const uint32_t (&v)[N], uint32_t active) {
  global_u32* w[N];
  int sh[N];
  uint32_t old[N];
  uint32_t pending = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p[i]);
    w[i] = global_dword(a);
    sh[i] = (a & 2) ? 16 : 0;
    old[i] = 0;
    if ((active >> i) & 1u) old[i] = __hip_atomic_load(w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (((active >> i) & 1u) && ((old[i] >> sh[i]) & 0xFFFFu) < v[i]) pending |= 1u << i;
  while (pending) {
    uint32_t prev[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((pending >> i) & 1u)
        prev[i] = global_cas(w[i], old[i], (old[i] & ~(0xFFFFu << sh[i])) | (v[i] << sh[i]));
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (!((pending >> i) & 1u)) continue;
      if (prev[i] == old[i] || ((prev[i] >> sh[i]) & 0xFFFFu) >= v[i])
        pending &= ~(1u << i);
      else
        old[i] = prev[i];
    }
  }
}

// Two BF16 entries sharing the aligned 32-bit word w (v: the low entry's value in bits 0-15, the
// high one's in 16-31).  Half h takes its value when its mode is 1 (the piece holds the block
// whole: set) or the max of its value and the word's when 2 (a block a fragment boundary cuts:
// merged); mode 0 leaves it alone.  Without a merge the halves are stored.  With one, a single
// thread owns the word, so no swap of this tile races another of its own; amax buffers are
// zero-filled before an update, so the first swap assumes a zero word, and any other value
// costs one retry with the word it found.
__device__ __forceinline__ void update_entry_pair(uint32_t* w, uint32_t v, int m0, int m1) {
  if (m0 != 2 && m1 != 2) {
    if (m0 && m1)
      *w = v;
    else if (m0)
      *reinterpret_cast<uint16_t*>(w) = (uint16_t)v;
    else if (m1)
      *(reinterpret_cast<uint16_t*>(w) + 1) = (uint16_t)(v >> 16);
    return;
  }
  uint32_t old = 0;
  bool known = false;  // old is the word's value, not the zero-fill guess
  for (;;) {
    const uint32_t lo = old & 0xFFFFu, hi = old >> 16;
    const uint32_t vl = v & 0xFFFFu, vh = v >> 16;
    const uint32_t nl = m0 == 1 ? vl : (m0 == 2 ? umax(lo, vl) : lo);
    const uint32_t nh = m1 == 1 ? vh : (m1 == 2 ? umax(hi, vh) : hi);
    const uint32_t nw = nl | (nh << 16);
    if (known && nw == old) return;
    const uint32_t prev = global_cas(global_dword(reinterpret_cast<uintptr_t>(w)), old, nw);
    if (prev == old) return;
    old = prev;
    known = true;
  }
}

// Entry words: BF16 entry updates planned ahead of the data (the amax's narrow edge tiles).  An
// entry is updated through the aligned 32-bit word that holds two of them.  An EntryWord names
// that word and, per half h (bits 16h .. 16h + 15 of v), whether to store it (bit h of `set`:
// the piece holds the block whole, so this thread is its only writer) or MAX-merge it (bit h
// of `merge`: a fragment boundary cuts the block, so a neighbouring piece may share it).
// Halves in neither mask are left alone.
struct EntryWord {
  uint32_t* w;
  uint32_t v;
  uint32_t set, merge;
};

// Half h of the word's value (0: none) for a lone entry p, with mode 1 (store) or 2 (merge).
__device__ __forceinline__ EntryWord entry_half(uint16_t* p, uint32_t v, int mode) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const int h = (int)(a >> 1) & 1;
  return EntryWord{reinterpret_cast<uint32_t*>(a & ~uintptr_t(3)), v << (16 * h),
                   (uint32_t)(mode == 1) << h, (uint32_t)(mode == 2) << h};
}

// Both halves of the aligned word w (v: the low entry's value in bits 0-15, the high one's in
// 16-31), with modes m0, m1 as for entry_half.
__device__ __forceinline__ EntryWord entry_pair(uint16_t* w, uint32_t v, int m0, int m1) {
  return EntryWord{reinterpret_cast<uint32_t*>(w), v,
                   (uint32_t)(m0 == 1) | ((uint32_t)(m1 == 1) << 1),
                   (uint32_t)(m0 == 2) | ((uint32_t)(m1 == 2) << 1)};
}

// The word that results from `old` under u.
__device__ __forceinline__ uint32_t entry_word_update(uint32_t old, const EntryWord& u) {
  uint32_t out = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t o = (old >> (16 * h)) & 0xFFFFu, v = (u.v >> (16 * h)) & 0xFFFFu;
    const uint32_t n = ((u.set >> h) & 1u) ? v : (((u.merge >> h) & 1u) ? umax(o, v) : o);
    out |= n << (16 * h);
  }
  return out;
}

// Applies N entry words atomically, old[i] being a value of word i read earlier in the
// launch.  Words without a merge are plain stores (32 or 16 bits).  The others go through
// compare-and-swap expecting old[i], all issued before any result is awaited, so they cost one
// round trip together; a word that already holds the result is left alone, and a swap that
// finds another value (a neighbouring piece's merge, an entry of the word stored by another
// thread) retries with it.
template <int N>
__device__ __forceinline__ void apply_entry_words(const EntryWord (&u)[N],
                                                  const uint32_t (&old0)[N]) {
  uint32_t old[N], pending = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    old[i] = old0[i];
    if (u[i].merge) {
      pending |= 1u << i;
    } else if (u[i].set == 3u) {
      *u[i].w = u[i].v;
    } else if (u[i].set == 1u) {
      *reinterpret_cast<uint16_t*>(u[i].w) = (uint16_t)u[i].v;
    } else if (u[i].set == 2u) {
      *(reinterpret_cast<uint16_t*>(u[i].w) + 1) = (uint16_t)(u[i].v >> 16);
    }
  }
  while (pending) {
    uint32_t prev[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      prev[i] = old[i];
      if (!((pending >> i) & 1u)) continue;
      const uint32_t nw = entry_word_update(old[i], u[i]);
      if (nw == old[i])
        pending &= ~(1u << i);  // the word already holds the result
      else
        prev[i] = global_cas(global_dword(reinterpret_cast<uintptr_t>(u[i].w)), old[i], nw);
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (((pending >> i) & 1u) && prev[i] == old[i]) pending &= ~(1u << i);
#pragma unroll
    for (int i = 0; i < N; ++i) old[i] = prev[i];
  }
}

// Applies N entry words with plain stores, merges taken against old[i], the word's value at
// the start of the launch: for a piece that no other piece of its launch shares amax arrays
// with, every entry has one writer in the launch, and a launch runs after the work enqueued
// before it.  Only the halves a word updates are stored.
template <int N>
__device__ __forceinline__ void store_entry_words(const EntryWord (&u)[N],
                                                  const uint32_t (&old)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t act = u[i].set | u[i].merge;
    const uint32_t nw = entry_word_update(old[i], u[i]);
    if (act == 3u)
      *u[i].w = nw;
    else if (act == 1u)
      *reinterpret_cast<uint16_t*>(u[i].w) = (uint16_t)nw;
    else if (act == 2u)
      *(reinterpret_cast<uint16_t*>(u[i].w) + 1) = (uint16_t)(nw >> 16);
  }
}

// The entry of a block: set when the piece holds the whole block (`whole`: its only writer),
// else MAX-merged atomically (a neighbouring piece may share the block).
template <typename T>
__device__ __forceinline__ void write_entry(void* base, int64_t idx, uint32_t v, bool whole) {
  T* p = static_cast<T*>(base) + idx;
  if (whole) {
    *p = (T)v;
  } else {
    T* const ps[1] = {p};
    const uint32_t vs[1] = {v};
    atomic_max_entries<1>(ps, vs, 1u);
  }
}

// ------------------------------------------------------------------ per-element working values

// |w| as the amax bit pattern, for one element given by its raw input bits.
template <typename T, bool kPre>
__device__ __forceinline__ uint32_t abs_bits(uint32_t raw) {
  if constexpr (sizeof(T) == 2) {
    return raw & 0x7FFFu;
  } else {
    return (kPre ? round_bf16_bits(raw) : raw) & 0x7FFFFFFFu;
  }
}

template <typename T, bool kPre>
__device__ __forceinline__ float work_value(uint32_t raw) {
  if constexpr (sizeof(T) == 2) {
    return __uint_as_float(raw << 16);
  } else {
    return __uint_as_float(kPre ? round_bf16_bits(raw) : raw);
  }
}

// Two working values -> two E4M3 bytes in the low or high half of `old`.
template <bool kHigh>
__device__ __forceinline__ uint32_t cvt2(float a, float b, int exp_shift_a, int exp_shift_b,
                                         uint32_t old) {
  float ya = __builtin_amdgcn_fmed3f(__builtin_ldexpf(a, exp_shift_a), -448.0f, 448.0f);
  float yb = __builtin_amdgcn_fmed3f(__builtin_ldexpf(b, exp_shift_b), -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, (int)old, kHigh);
}

__device__ __forceinline__ uint8_t cvt1(float a, int exp_shift) {
  float y = __builtin_amdgcn_fmed3f(__builtin_ldexpf(a, exp_shift), -448.0f, 448.0f);
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFF);
}

__device__ __forceinline__ uint32_t load_raw(const void* input, int64_t k, int esize) {
  return esize == 2 ? (uint32_t)static_cast<const uint16_t*>(input)[k]
                    : static_cast<const uint32_t*>(input)[k];
}

// ------------------------------------------------------------------ chunk helpers (vector path)

template <typename T>
struct Chunk {
  static constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
};

// Raw bits of element e of a chunk held as 4 dwords.
template <typename T>
__device__ __forceinline__ uint32_t chunk_elem(const uint32_t (&d)[4], int e) {
  if constexpr (sizeof(T) == 2)
    return (d[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
  else
    return d[e];
}

// Fold a chunk into the lane's column-wise maxima and return the chunk's own max |w|.
// BF16: col[j] packs columns 2j (low half) and 2j+1 (high half), the entries' memory order.
template <typename T, bool kCol, bool kPre>
__device__ __forceinline__ uint32_t chunk_absmax(const uint32_t (&d)[4], uint32_t (&col)[4]) {
  uint32_t a[4];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = d[j] & 0x7FFF7FFFu;
      if constexpr (kCol) col[j] = pk_max_u16(col[j], a[j]);
    }
    const uint32_t m = pk_max_u16(pk_max_u16(a[0], a[1]), pk_max_u16(a[2], a[3]));
    return umax(m & 0xFFFFu, m >> 16);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = (kPre ? round_bf16_bits(d[j]) : d[j]) & 0x7FFFFFFFu;
      if constexpr (kCol) col[j] = umax(col[j], a[j]);
    }
    return umax(umax(a[0], a[1]), umax(a[2], a[3]));
  }
}

// Column-wise amax of column e of the chunk from the packed maxima.
template <typename T>
__device__ __forceinline__ uint32_t col_entry(const uint32_t (&col)[4], int e) {
  if constexpr (sizeof(T) == 2)
    return (col[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
  else
    return col[e];
}

__device__ __forceinline__ void load16(const void* p, uint32_t (&d)[4]) {
  const uint4 v = *static_cast<const uint4*>(p);
  d[0] = v.x;
  d[1] = v.y;
  d[2] = v.z;
  d[3] = v.w;
}

// Vector types that need only dword alignment: for accesses of a dword or more the hardware
// ignores the two low address bits, so a 16-byte load from any 4-byte-aligned address is one
// global_load_dwordx4 (a fragment's chunks are 16-byte aligned only when input - start is).
typedef unsigned int v4u __attribute__((ext_vector_type(4), aligned(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2), aligned(4)));

// The input is streamed once: non-temporal loads (the "nt" cache policy) keep it from
// displacing reused lines; on MI355X they also lift a pure read stream from ~5.9 to ~6.7 TB/s.
//
// A chunk is loaded in two steps, issue_chunk and then assemble_chunk, so that a wave issues
// the loads of all its rows before it uses (and so waits for) any of them: a use inside the
// branch that loads a row makes the compiler wait there, one round trip per row.
struct RawChunk {
  v4u v;
  uint32_t t;
};

// The 16 bytes at p.  With shift2 (BF16 input whose input - start sits at 2 mod 4) p is 2
// bytes past a dword boundary: the dword-aligned 16 bytes before it plus the next dword are
// loaded instead.  The extra 2 bytes on each side lie in the same dwords as the chunk's first
// and last element.
__device__ __forceinline__ void issue_chunk(const void* p, bool shift2, RawChunk& r) {
  if (shift2) {
    const uint8_t* b = static_cast<const uint8_t*>(p) - 2;
    r.v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(b));
    r.t = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(b + 16));
  } else {
    r.v = __builtin_nontemporal_load(static_cast<const v4u*>(p));
    r.t = 0;
  }
}

__device__ __forceinline__ void assemble_chunk(const RawChunk& r, bool shift2, uint32_t (&d)[4]) {
  if (shift2) {
    d[0] = __builtin_amdgcn_alignbyte(r.v.y, r.v.x, 2);
    d[1] = __builtin_amdgcn_alignbyte(r.v.z, r.v.y, 2);
    d[2] = __builtin_amdgcn_alignbyte(r.v.w, r.v.z, 2);
    d[3] = __builtin_amdgcn_alignbyte(r.t, r.v.w, 2);
  } else {
    d[0] = r.v.x;
    d[1] = r.v.y;
    d[2] = r.v.z;
    d[3] = r.v.w;
  }
}

// Chunks src + i * cols, i < n (n <= RW; the others stay as they are): all loads are issued
// before any is assembled.  With shift2 and `whole_wave` (every lane of the wave is active and
// the 64 lanes hold consecutive chunks of each row), the dword after a lane's 16 bytes is the
// next lane's first dword: lanes take it from their neighbour with a DPP wave shift, and only
// lane 63's, one uniform address per row (the dword its own shifted load would read), is
// loaded, in place of a scattered extra dword load per lane and row.
template <typename T, int RW>
__device__ __forceinline__ void load_rows(const T* src, int64_t cols, bool shift2, int n,
                                          uint32_t (&d)[RW][4], bool whole_wave) {
  RawChunk raw[RW];
  if (shift2 && whole_wave) {
    const uint64_t a = reinterpret_cast<uint64_t>(src);
    const uint64_t a63 =
        ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(a >> 32), kWaveSize - 1) << 32) |
        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)a, kWaveSize - 1);
    // lane 63's next dword (p + 14 for a chunk at p = 2 mod 4: dword-aligned).  The mask keeps
    // the compiler from folding the 14 into the instruction offset of a scalar load, whose
    // hardware drops the two low bits of the base address before adding the offset.
    const uint64_t t63 = a63 + 14;
    uint32_t tail[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if (i < n) {
        raw[i].v = __builtin_nontemporal_load(
            reinterpret_cast<const v4u*>(reinterpret_cast<const uint8_t*>(src + i * cols) - 2));
        tail[i] = *global_cdword(t63 + i * cols * (int64_t)sizeof(T));
      }
    }
    const bool top = (threadIdx.x & (kWaveSize - 1)) == kWaveSize - 1;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if (i < n) {
        // wave_shl:1 (DPP control 0x130): lane l reads lane l + 1; lane 63 keeps `old`
        const uint32_t next = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)raw[i].v.x, 0x130,
                                                                    0xF, 0xF, false);
        raw[i].t = top ? tail[i] : next;
        assemble_chunk(raw[i], true, d[i]);
      }
    }
  } else if (shift2) {
#pragma unroll
    for (int i = 0; i < RW; ++i)
      if (i < n) issue_chunk(src + i * cols, true, raw[i]);
#pragma unroll
    for (int i = 0; i < RW; ++i)
      if (i < n) assemble_chunk(raw[i], true, d[i]);
  } else {
#pragma unroll
    for (int i = 0; i < RW; ++i)
      if (i < n) issue_chunk(src + i * cols, false, raw[i]);
#pragma unroll
    for (int i = 0; i < RW; ++i)
      if (i < n) assemble_chunk(raw[i], false, d[i]);
  }
}

// Chunk g's elements in `mask` (a chunk that a fragment boundary cuts; 0: no such chunk), as
// raw dwords for assemble_chunk: the dwords of the chunk's window (4, or 5 for a BF16 input 2
// bytes off a dword) that hold an element of the mask are loaded; every other dword re-reads
// the first of those (dropped by masked_chunk), and without a mask all of them read the dword
// holding the fragment's first element.  A load never reaches a dword without an element of the
// fragment, so it stays inside the caller's allocation.  The loads go out unconditionally: a load
// under a per-lane condition lets the compiler place the first use of its value, and with it a
// wait for every load in flight, inside the condition.
template <typename T>
__device__ __forceinline__ void issue_masked(const TileArgs& p, int64_t g, uint32_t mask,
                                             RawChunk& r) {
  const bool s2 = sizeof(T) == 2 && p.in_shift2;
  const uint8_t* a =
      static_cast<const uint8_t*>(p.input) + (mask ? (g - p.start) * (int64_t)sizeof(T) : 0);
  global_cu32* w = global_cdword(reinterpret_cast<uintptr_t>(a));
  uint32_t hold = 0;  // bit j: dword j of the window holds an element of the mask
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    uint32_t el;  // the elements dword j holds
    if constexpr (sizeof(T) == 4)
      el = j < 4 ? 1u << j : 0u;
    else
      el = s2 ? (3u << (2 * j)) >> 1 : (j < 4 ? 3u << (2 * j) : 0u);
    hold |= (mask & el) ? 1u << j : 0u;
  }
  const int jf = hold ? __builtin_ctz(hold) : 0;
  uint32_t v[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) v[j] = (j < 4 || s2) ? w[((hold >> j) & 1u) ? j : jf] : 0u;
  r.v = v4u{v[0], v[1], v[2], v[3]};
  r.t = v[4];
}

// The assembled chunk d with the elements outside `mask` set to 0.
template <typename T>
__device__ __forceinline__ void masked_chunk(uint32_t mask, uint32_t (&d)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (sizeof(T) == 2)
      d[j] &= (((mask >> (2 * j)) & 1u) ? 0xFFFFu : 0u) |
              (((mask >> (2 * j + 1)) & 1u) ? 0xFFFF0000u : 0u);
    else
      d[j] = ((mask >> j) & 1u) ? d[j] : 0u;
  }
}

// Which of an edge tile's rows hold a whole chunk of the fragment, which (at most two: the
// fragment's start and end) a chunk that a fragment boundary cuts, and each row's element
// mask; from the bounds alone, so a caller can issue other loads before the rows'.
template <int RW>
struct RowClass {
  uint32_t full;      // bit i: row i's chunk lies wholly inside the fragment
  int cut0, cut1;     // rows whose chunk a fragment boundary cuts (-1: none)
  uint32_t m0, m1;    // their element masks (0: none)
  uint32_t em[RW];    // element masks of all rows
};

// Element mask of chunk g within [start, end).
template <int E>
__device__ __forceinline__ uint32_t chunk_mask(const TileArgs& p, int64_t g) {
  const int lo = (int)max<int64_t>(0, min<int64_t>(E, p.start - g));  // first element inside
  const int hi = (int)max<int64_t>(0, min<int64_t>(E, p.end - g));    // one past the last
  return ((1u << hi) - 1) & ~((1u << lo) - 1);
}

// Rows i < nrows_here of the wave, chunk column c.  Chunks start at flat indices congruent to
// p.shift modulo E (0 except in the line-owned cast tiles); c may then pass the row's end.
template <typename T, int RW>
__device__ __forceinline__ RowClass<RW> classify_rows(const TileArgs& p, int64_t rfirst,
                                                      int nrows_here, int64_t c, bool cvalid) {
  constexpr int E = Chunk<T>::E;
  RowClass<RW> k;
  k.full = 0;
  k.cut0 = k.cut1 = -1;
  k.m0 = k.m1 = 0;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    k.em[i] = 0;
    if (i < nrows_here && cvalid) {
      const int64_t g = (rfirst + i) * p.cols + c;
      if (g >= p.start && g + E <= p.end) {
        k.full |= 1u << i;
        k.em[i] = (1u << E) - 1;
      } else if (g + E > p.start && g < p.end) {
        k.em[i] = chunk_mask<E>(p, g);
        if (k.cut0 < 0) {
          k.cut0 = i;
          k.m0 = k.em[i];
        } else {
          k.cut1 = i;
          k.m1 = k.em[i];
        }
      }
    }
  }
  return k;
}

// Rows of an edge tile (as classified), masked to the fragment, in d (elements outside it
// are 0).  The whole chunks' loads go out first, then the word loads of the cut chunks, and
// only then is anything assembled.
template <typename T, int RW>
__device__ __forceinline__ void load_rows_masked(const TileArgs& p, const T* src, int64_t rfirst,
                                                 int64_t c, const RowClass<RW>& k,
                                                 uint32_t (&d)[RW][4]) {
  constexpr int E = Chunk<T>::E;
  // Every lane issues every row's chunk load, rows without a whole chunk reading the
  // fragment's first whole chunk instead (discarded): a load under a per-lane condition would
  // make the compiler wait for it where the branches join.  That chunk starts at the first
  // chunk start at or after start (chunks start on one grid of the flat index, since
  // cols % E == 0), so its load touches only what a whole chunk's load touches; it is not
  // input itself, which with a 2-byte shift would read the 2 bytes before the fragment, in
  // another dword.  A fragment without a whole chunk loads nothing.
  RawChunk raw[RW];
  const int64_t g_whole = p.start + ((((int64_t)p.shift - p.start) % E) + E) % E;
  if (g_whole + E <= p.end) {
    const T* whole = static_cast<const T*>(p.input) + (g_whole - p.start);
#pragma unroll
    for (int i = 0; i < RW; ++i)
      issue_chunk(((k.full >> i) & 1u) ? src + i * p.cols : whole, p.in_shift2, raw[i]);
  }
  RawChunk cr0, cr1;
  issue_masked<T>(p, (rfirst + max(k.cut0, 0)) * p.cols + c, k.m0, cr0);
  issue_masked<T>(p, (rfirst + max(k.cut1, 0)) * p.cols + c, k.m1, cr1);
  uint32_t c0d[4], c1d[4];
  assemble_chunk(cr0, p.in_shift2, c0d);
  assemble_chunk(cr1, p.in_shift2, c1d);
  masked_chunk<T>(k.m0, c0d);
  masked_chunk<T>(k.m1, c1d);
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const bool whole = (k.full >> i) & 1u;
    assemble_chunk(raw[i], p.in_shift2, d[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d[i][j] = whole ? d[i][j] : 0u;
      d[i][j] = i == k.cut0 ? c0d[j] : d[i][j];
      d[i][j] = i == k.cut1 ? c1d[j] : d[i][j];
    }
  }
}

// The row classification of the amax's narrow edge tiles (8 waves of 4 rows), where the tile's
// latency is the call's: as RowClass without the per-row masks (cut_mask derives them), and
// computed without branches, so the rows' loads go out soon after the tile starts; the loads
// are issued (issue_rows_masked) and assembled (assemble_rows_masked) apart, so the caller can
// do what needs no data in between.
template <int RW>
struct RowCuts {
  uint32_t full;      // bit i: row i's chunk lies wholly inside the fragment
  int cut0, cut1;     // rows whose chunk a fragment boundary cuts (-1: none)
  uint32_t m0, m1;    // their element masks (0: none)
};

// Row i's element mask (bit e: element e of its chunk lies in the fragment).
template <typename T, int RW>
__device__ __forceinline__ uint32_t cut_mask(const RowCuts<RW>& k, int i) {
  constexpr uint32_t kAll = (1u << Chunk<T>::E) - 1;
  return ((k.full >> i) & 1u) ? kAll : (i == k.cut0 ? k.m0 : (i == k.cut1 ? k.m1 : 0u));
}

// Rows i < nrows_here of the wave, chunk column c (as classify_rows).
template <typename T, int RW>
__device__ __forceinline__ RowCuts<RW> classify_cuts(const TileArgs& p, int64_t rfirst,
                                                     int nrows_here, int64_t c, bool cvalid) {
  constexpr int E = Chunk<T>::E;
  RowCuts<RW> k;
  k.full = 0;
  k.cut0 = k.cut1 = -1;
  const int64_t g0 = rfirst * p.cols + c;  // the first row's chunk
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int64_t g = g0 + i * p.cols;
    const bool in = (i < nrows_here) & cvalid;
    const bool whole = in & (g >= p.start) & (g + E <= p.end);
    const bool cut = in & !whole & (g + E > p.start) & (g < p.end);
    k.full |= (uint32_t)whole << i;
    // a chunk column meets the fragment's two boundaries at most once each
    const bool first = cut & (k.cut0 < 0);
    const bool second = cut & !first;
    k.cut1 = second ? i : k.cut1;
    k.cut0 = first ? i : k.cut0;
  }
  // the cut chunks' masks: elements [lo, hi) of the chunk lie in the fragment (both in [0, E]
  // for a cut chunk; for none the mask is 0)
  auto mask = [&](int i) -> uint32_t {
    const int64_t g = g0 + max(i, 0) * p.cols;
    const int lo = g < p.start ? (int)(p.start - g) : 0;
    const int hi = g + E > p.end ? (int)(p.end - g) : E;
    const uint32_t m = ((1u << (hi & 31)) - 1) & ~((1u << (lo & 31)) - 1);
    return i >= 0 ? m : 0u;
  };
  k.m0 = mask(k.cut0);
  k.m1 = mask(k.cut1);
  return k;
}

// The loads of an edge tile's rows in flight.
template <int RW>
struct MaskedRows {
  RawChunk raw[RW];
  RawChunk cr0, cr1;
};

// Issues the rows' loads as load_rows_masked does: the whole chunks' first (one uniform branch
// on the 2-byte shift for all rows), then the word loads of the cut chunks.
template <typename T, int RW>
__device__ __forceinline__ void issue_rows_masked(const TileArgs& p, const T* src, int64_t rfirst,
                                                  int64_t c, const RowCuts<RW>& k,
                                                  MaskedRows<RW>& ml) {
  constexpr int E = Chunk<T>::E;
  const int64_t g_whole = p.start + ((((int64_t)p.shift - p.start) % E) + E) % E;
  if (g_whole + E <= p.end) {
    const T* whole = static_cast<const T*>(p.input) + (g_whole - p.start);
    if (sizeof(T) == 2 && p.in_shift2) {
#pragma unroll
      for (int i = 0; i < RW; ++i)
        issue_chunk(((k.full >> i) & 1u) ? src + i * p.cols : whole, true, ml.raw[i]);
    } else {
#pragma unroll
      for (int i = 0; i < RW; ++i)
        issue_chunk(((k.full >> i) & 1u) ? src + i * p.cols : whole, false, ml.raw[i]);
    }
  }
  issue_masked<T>(p, (rfirst + max(k.cut0, 0)) * p.cols + c, k.m0, ml.cr0);
  issue_masked<T>(p, (rfirst + max(k.cut1, 0)) * p.cols + c, k.m1, ml.cr1);
}

// The rows in d, masked to the fragment (elements outside it are 0).
template <typename T, int RW>
__device__ __forceinline__ void assemble_rows_masked(const TileArgs& p, const RowCuts<RW>& k,
                                                     const MaskedRows<RW>& ml,
                                                     uint32_t (&d)[RW][4]) {
  const bool s2 = sizeof(T) == 2 && p.in_shift2;
  uint32_t c0d[4], c1d[4];
  assemble_chunk(ml.cr0, s2, c0d);
  assemble_chunk(ml.cr1, s2, c1d);
  masked_chunk<T>(k.m0, c0d);
  masked_chunk<T>(k.m1, c1d);
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const bool whole = (k.full >> i) & 1u;
    assemble_chunk(ml.raw[i], s2, d[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d[i][j] = whole ? d[i][j] : 0u;
      d[i][j] = i == k.cut0 ? c0d[j] : d[i][j];
      d[i][j] = i == k.cut1 ? c1d[j] : d[i][j];
    }
  }
}

// Scale byte from the amax bit pattern: floor(log2 amax) = exponent field - 127 for normal
// values, so the biased MX exponent is field - 8, clamped at 0 (subnormal and zero amax
// included); the field is at most 254 for finite amax, so the upper clamp never applies.
template <typename T>
__device__ __forceinline__ uint8_t e8m0_of(uint32_t bits) {
  const int field = sizeof(T) == 2 ? (int)((bits >> 7) & 0xFF) : (int)((bits >> 23) & 0xFF);
  return (uint8_t)(field > 8 ? field - 8 : 0);
}

// Whether row-wise block (r, c / 32) holds an element of the fragment (any width of row).
__device__ __forceinline__ bool row_block_touched(const TileArgs& p, int64_t r, int64_t c) {
  const int64_t gb = r * p.cols + (c & ~int64_t(kBlockLen - 1));
  const int64_t ge = min<int64_t>(gb + kBlockLen, (r + 1) * p.cols);
  return gb < p.end && ge > p.start;
}

// Row and column of the fragment's first and last element.
struct Corners {
  int64_t rs, cs, re, ce;
};
__device__ __forceinline__ Corners corners_of(const TileArgs& p) {
  Corners f;
  f.rs = p.start / p.cols;
  f.cs = p.start - f.rs * p.cols;
  f.re = (p.end - 1) / p.cols;
  f.ce = p.end - 1 - f.re * p.cols;
  return f;
}

// Whether the column-wise block of rows [r0, r1] in column col holds an element of the
// fragment: the fragment's rows in column col run from rs (rs + 1 left of cs) to re (re - 1
// right of ce).
__device__ __forceinline__ bool col_block_touched(const Corners& f, int64_t r0, int64_t r1,
                                                  int64_t col) {
  const int64_t lo = max(r0, col >= f.cs ? f.rs : f.rs + 1);
  const int64_t hi = min(r1, col <= f.ce ? f.re : f.re - 1);
  return lo <= hi;
}

// ------------------------------------------------------------------ partial amax, vector path

constexpr int kRowsPerWave = kBlockLen / kWavesPerGroup;  // 8 rows of the band per wave

template <typename T>
__device__ __forceinline__ void fold_col(uint32_t (&col)[4], const uint4& o) {
  const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) col[j] = sizeof(T) == 2 ? pk_max_u16(col[j], ov[j]) : umax(col[j], ov[j]);
}

// A workgroup owns one tile: a 32-row band x 64*E columns.  Wave w streams rows 8w .. 8w+7
// with all eight 16-byte loads in flight; the four waves' column-wise maxima meet in LDS.
// Tiles wholly inside the fragment write their entries without reading them (each block has
// a single owner); edge tiles write the entries of blocks the piece holds whole and merge
// those of cut blocks atomically, since a neighbouring piece may share them.
// kGuard (with kCol = true; the ablation library, and small calls holding both directions):
// one kernel for both kinds of piece, its column-wise work selected at run time by the
// column-wise pointer.  kWaves: the workgroup's waves, each taking 32 / kWaves rows of the
// band (8 waves of 4 rows for launches too small to fill the GPU).  kOne: a launch of a single
// piece (Tier::one), whose piece index is 0.
template <typename T, bool kCol, bool kPre, int kOcc, bool kGuard = false,
          int kWaves = kWavesPerGroup, bool kOne = false>
__global__ __launch_bounds__(kWaveSize * kWaves)
__attribute__((amdgpu_waves_per_eu(kOcc))) void amax_vec_kernel(GroupArgs ga) {
  constexpr int E = Chunk<T>::E;
  constexpr int LB = kBlockLen / E;     // lanes sharing one row-wise block (4 BF16, 8 FP32)
  constexpr int WC = kWaveSize * E;     // tile width in columns
  constexpr int RW = kBlockLen / kWaves;  // rows of the band per wave (8; 4 with 8 waves)
  constexpr int NK = RW >= LB ? RW / LB : 1;  // row maxima each lane keeps (2 BF16, 1 FP32)
  constexpr int NBLK = WC / kBlockLen;  // row-wise blocks across the tile (16 BF16, 8 FP32)
  constexpr int kT = kWaveSize * kWaves;  // threads of the workgroup
  __shared__ uint4 s_col[kWaves][kWaveSize];
  __shared__ uint32_t s_touch[kWaves][kWaveSize];
  __shared__ uint32_t s_rmax[kBlockLen][NBLK];

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = threadIdx.x >> 6;
  if constexpr (!kOne) pin_header(ga);
  const uint32_t lt = xcd_remap(blockIdx.x, gridDim.x);  // tile of the launch
  const int k = kOne ? 0 : piece_of(ga, lt);  // a launch of one piece: piece 0
  const TileArgs& p = ga.piece[k];
  pin_tile_fields(ga, k);
  const int64_t tile = (int64_t)(lt - ga.first[k]) + p.tile0;
  if (tile >= p.ntiles) return;  // uniform over the workgroup
  const uint32_t t32 = (uint32_t)tile, n32 = (uint32_t)p.ntc, bq = t32 / n32;
  const int64_t band = p.band0 + bq;
  const int64_t c0 = (int64_t)(t32 - bq * n32) * WC;
  const int64_t c = c0 + lane * E;
  const int64_t r0 = band * kBlockLen;
  const bool cvalid = c < p.cols;
  const int nrows = (int)min<int64_t>(kBlockLen, p.rows - r0);
  const int i0 = wave * RW;  // this wave's first row within the band
  const int64_t tile_first = r0 * p.cols + c0;
  const int64_t tile_end = (r0 + nrows - 1) * p.cols + min<int64_t>(c0 + WC, p.cols);
  // A tile holding a row's short last block (cols % 32 != 0) takes the edge path, whose entry
  // writes go through LDS: the interior path's per-lane writes assume whole blocks.  The tests
  // are joined with & rather than &&: every field they read is then loaded in one batch, where
  // a branch per test cost a scalar round trip each before the tile's first global load.
  const bool interior = (nrows == kBlockLen) & (tile_first >= p.start) & (tile_end <= p.end) &
                        ((p.cols % kBlockLen == 0) | (c0 + WC <= p.cols));
  const bool colw = kCol && (!kGuard || p.amax_col != nullptr);  // column-wise entries

  uint32_t col[4] = {0, 0, 0, 0};
  uint32_t d[RW][4];
  const T* src = static_cast<const T*>(p.input) + ((r0 + i0) * p.cols + c - p.start);

  if (interior) {
#pragma unroll
    for (int i = 0; i < RW; ++i) d[i][0] = d[i][1] = d[i][2] = d[i][3] = 0;
    if (cvalid) load_rows<T, RW>(src, p.cols, p.in_shift2, RW, d, c0 + WC <= p.cols);
    // Entries of the tile: 32 rows x NBLK row-wise blocks (32 bytes per row) and 64*E
    // column-wise blocks, all held whole by this piece, so they are written and never read.
    // Wave 1 writes the row-wise entries as one 16-byte vector per lane (row lane/2, half
    // lane%2) while wave 0 combines and writes the column-wise ones.  Tiles whose rows are not
    // 16-byte aligned in amax_row, or that run past the last column, let every block's owner
    // lanes write their entries one by one.
    constexpr int EPV = 16 / (int)sizeof(T);  // entries per 16-byte vector (NBLK = 2 * EPV)
    const bool rvec = p.row_vec && c0 + WC <= p.cols;  // uniform
    T* ar = static_cast<T*>(p.amax_row) + (r0 + i0 + lane % LB) * p.ld_ar + (c >> 5);
    T* arv = static_cast<T*>(p.amax_row) + (r0 + (lane >> 1)) * p.ld_ar + (c0 >> 5) +
             (lane & 1) * EPV;
    T* ac = static_cast<T*>(p.amax_col) + band * p.ld_ac + c;
    uint32_t keep[NK];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      uint32_t m = chunk_absmax<T, kCol, kPre>(d[i], col);
      m = group_max<LB>(m);
      if (rvec) {
        if ((lane % LB) == 0) s_rmax[i0 + i][lane / LB] = m;
      } else if ((i % LB) == (lane % LB)) {
        keep[i / LB] = m;
      }
    }
    // (with fewer rows per wave than lanes per block, lane l keeps row l % LB if it has one)
    if (!rvec && cvalid && (RW >= LB || lane % LB < RW)) {
#pragma unroll
      for (int k = 0; k < NK; ++k) ar[(int64_t)k * LB * p.ld_ar] = (T)keep[k];
    }
    if (colw) s_col[wave][lane] = make_uint4(col[0], col[1], col[2], col[3]);
    if (rvec || colw) __syncthreads();
    if (rvec && wave == 1) {
      uint32_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(T) == 2)
          v[j] = s_rmax[lane >> 1][(lane & 1) * EPV + 2 * j] |
                 (s_rmax[lane >> 1][(lane & 1) * EPV + 2 * j + 1] << 16);
        else
          v[j] = s_rmax[lane >> 1][(lane & 1) * EPV + j];
      }
      *reinterpret_cast<uint4*>(arv) = make_uint4(v[0], v[1], v[2], v[3]);
    }
    if (colw) {
      if (wave == 0 && cvalid) {
#pragma unroll
        for (int w = 1; w < kWaves; ++w) fold_col<T>(col, s_col[w][lane]);
        if (p.col_vec) {
          *reinterpret_cast<uint4*>(ac) = make_uint4(col[0], col[1], col[2], col[3]);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) ac[e] = (T)col_entry<T>(col, e);
        }
      }
    }
    return;
  }

  if constexpr (kWaves >= 8 && sizeof(T) == 2) {
    // BF16 edge tile of a launch too small to fill the GPU, whose latency is the call's.  As
    // below, but each thread (of 512) takes one row-wise and one column-wise entry word, planned
    // from the geometry alone while the rows' loads are in flight: a word that takes a merge is
    // loaded with the data (a word without one loads the tile's first row-wise entry word
    // instead, so every load stays in bounds).  A piece that owns its amax arrays in the launch
    // then stores its merges against those values, and no compare-and-swap round trip follows
    // the data; otherwise the merges go through compare-and-swap, starting from them.
    static_assert(kBlockLen * NBLK <= kT && WC <= kT, "one entry of each kind per thread");
    const RowCuts<RW> rc = classify_cuts<T, RW>(p, r0 + i0, nrows - i0, c, cvalid);
    MaskedRows<RW> ml;
    issue_rows_masked<T, RW>(p, src, r0 + i0, c, rc, ml);
    // Which update a block's entry takes: 0 none (no element of the fragment), 1 a store (the
    // piece holds the block whole), 2 a merge (a fragment boundary cuts it).  A column-wise
    // block's mode holds if the column has an element of the fragment in the band.
    auto row_mode = [&](int row, int blk) -> int {
      const int64_t r = r0 + row;
      const int64_t bc = c0 + blk * kBlockLen;  // the block's first column
      const int64_t gb = r * p.cols + bc;
      const int64_t ge = r * p.cols + min<int64_t>(bc + kBlockLen, p.cols);  // one past it
      if (!(row < nrows && bc < p.cols && gb < p.end && ge > p.start)) return 0;
      return (gb >= p.start && ge <= p.end) ? 1 : 2;
    };
    auto col_mode = [&](int cc) -> int {
      const int64_t cg = c0 + cc;
      // the block's first and last elements decide whether the piece holds it whole
      const int64_t gf = r0 * p.cols + cg, gl = (r0 + nrows - 1) * p.cols + cg;
      if (cg >= p.cols) return 0;
      return (gf >= p.start && gl < p.end) ? 1 : 2;
    };
    constexpr int PR = NBLK / 2;  // BF16 entry words per row of the tile (8)
    const int t = threadIdx.x;
    T* const arow = static_cast<T*>(p.amax_row) + r0 * p.ld_ar + (c0 >> 5);
    T* const acol = static_cast<T*>(p.amax_col) + band * p.ld_ac + c0;
    // the thread's row-wise entry (or aligned pair: blocks 2k, 2k + 1) and column-wise column
    // (or aligned pair of columns 2t, 2t + 1); pairs where rows of the amax array start on
    // 4-byte boundaries, so no two threads of the tile share a word
    const bool rpair = p.row_pair, cpair = p.col_pair;
    const bool rok = t < kBlockLen * (rpair ? PR : NBLK);
    const int re = rok ? t : 0;
    const int row = rpair ? re / PR : re / NBLK;
    const int blk = rpair ? 2 * (re % PR) : re % NBLK;
    const int cc0 = cpair ? 2 * t : t;
    const bool cok = cc0 < WC;
    const int cc = cok ? cc0 : 0;
    EntryWord u[2];
    u[0] = rpair ? entry_pair(arow + row * p.ld_ar + blk, 0, rok ? row_mode(row, blk) : 0,
                              rok ? row_mode(row, blk + 1) : 0)
                 : entry_half(arow + row * p.ld_ar + blk, 0, rok ? row_mode(row, blk) : 0);
    u[1] = EntryWord{nullptr, 0, 0, 0};
    if (colw)
      u[1] = cpair ? entry_pair(acol + cc, 0, cok ? col_mode(cc) : 0, cok ? col_mode(cc + 1) : 0)
                   : entry_half(acol + cc, 0, cok ? col_mode(cc) : 0);
    const uintptr_t any = reinterpret_cast<uintptr_t>(arow);
    uint32_t old[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      old[j] = *global_cdword(u[j].merge ? reinterpret_cast<uintptr_t>(u[j].w) : any);

    assemble_rows_masked<T, RW>(p, rc, ml, d);
    uint32_t touched = 0;  // bit e: column c + e has an element of the fragment in these rows
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const uint32_t m = group_max<LB>(chunk_absmax<T, kCol, kPre>(d[i], col));
      if ((lane % LB) == 0) s_rmax[i0 + i][lane / LB] = m;
      touched |= cut_mask<T, RW>(rc, i);
    }
    s_col[wave][lane] = make_uint4(col[0], col[1], col[2], col[3]);
    s_touch[wave][lane] = touched;
    __syncthreads();

    // the column's (or pair's) maximum over the waves, and whether it has an element of the
    // fragment in the band
    const int ln = cc / E, e = cc % E;  // lane of s_col holding it, and its element there
    uint32_t cm = 0, ct = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint4 o = s_col[w][ln];
      const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
      cm = cpair ? pk_max_u16(cm, ov[e / 2]) : umax(cm, col_entry<T>(ov, e));
      ct |= s_touch[w][ln];
    }
    u[0].v = rpair ? s_rmax[row][blk] | (s_rmax[row][blk + 1] << 16)
                   : s_rmax[row][blk] << (((u[0].set | u[0].merge) & 2u) ? 16 : 0);
    if (cpair) {
      const uint32_t tm = (ct >> e) & 3u;  // e even: the pair's two columns
      u[1].v = cm;
      u[1].set &= tm;
      u[1].merge &= tm;
    } else {
      const int h = ((u[1].set | u[1].merge) & 2u) ? 1 : 0;  // the half holding the entry
      const uint32_t tm = ((ct >> e) & 1u) << h;
      u[1].v = cm << (16 * h);
      u[1].set &= tm;
      u[1].merge &= tm;
    }
    if (p.amax_own)
      store_entry_words(u, old);
    else
      apply_entry_words(u, old);
  } else {
    // Edge tile: a fragment boundary, the short last band or a row's short last block cuts it.
    // Every wave loads its rows masked to the fragment; the row-wise and column-wise maxima meet
    // in LDS and all threads then write the touched entries, at most two of each kind per
    // thread: blocks the piece holds whole are stored, blocks a fragment boundary cuts are
    // merged atomically (all reads, then all swaps).
    const RowClass<RW> rc = classify_rows<T, RW>(p, r0 + i0, nrows - i0, c, cvalid);
    const uint32_t(&em)[RW] = rc.em;
    load_rows_masked<T, RW>(p, src, r0 + i0, c, rc, d);
    uint32_t touched = 0;  // bit e: column c + e has an element of the fragment in these rows
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const uint32_t m = group_max<LB>(chunk_absmax<T, kCol, kPre>(d[i], col));
      if ((lane % LB) == 0) s_rmax[i0 + i][lane / LB] = m;
      touched |= em[i];
    }
    s_col[wave][lane] = make_uint4(col[0], col[1], col[2], col[3]);
    s_touch[wave][lane] = touched;
    __syncthreads();
    // BF16 entries whose rows start on 4-byte boundaries: one thread per aligned word of two
    // entries (row-wise: blocks 2k, 2k + 1 of a row; column-wise: columns 2t, 2t + 1)
    constexpr bool kPairs = sizeof(T) == 2;
    if (kPairs && p.row_pair && threadIdx.x < kBlockLen * (NBLK / 2)) {
      constexpr int PR = NBLK / 2;  // word pairs per row of the tile (8)
      const int row = threadIdx.x / PR, k2 = 2 * (threadIdx.x % PR);
      const int64_t r = r0 + row;
      int mode[2] = {0, 0};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t bc = c0 + (k2 + h) * kBlockLen;  // the block's first column
        const int64_t gb = r * p.cols + bc;
        const int64_t ge = r * p.cols + min<int64_t>(bc + kBlockLen, p.cols);  // one past its last
        if (row < nrows && bc < p.cols && gb < p.end && ge > p.start)
          mode[h] = (gb >= p.start && ge <= p.end) ? 1 : 2;
      }
      if (mode[0] | mode[1])
        update_entry_pair(reinterpret_cast<uint32_t*>(static_cast<T*>(p.amax_row) + r * p.ld_ar +
                                                      (c0 >> 5) + k2),
                          s_rmax[row][k2] | (s_rmax[row][k2 + 1] << 16), mode[0], mode[1]);
    } else {
      // row entries per thread (2 or 1 with 256 threads; threads past the tile's entries idle)
      constexpr int kPer = kBlockLen * NBLK >= kT ? kBlockLen * NBLK / kT : 1;
      T* ptr[kPer];
      uint32_t v[kPer], act = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int e0 = threadIdx.x + j * kT;
        const bool ok = e0 < kBlockLen * NBLK;
        const int e = ok ? e0 : 0;
        const int row = e / NBLK, blk = e % NBLK;
        const int64_t r = r0 + row;
        const int64_t bc = c0 + blk * kBlockLen;  // the block's first column
        const int64_t gb = r * p.cols + bc;
        const int64_t ge = r * p.cols + min<int64_t>(bc + kBlockLen, p.cols);  // one past its last
        ptr[j] = static_cast<T*>(p.amax_row) + r * p.ld_ar + (c0 >> 5) + blk;
        v[j] = s_rmax[row][blk];
        if (ok && row < nrows && bc < p.cols && gb < p.end && ge > p.start) {
          if (gb >= p.start && ge <= p.end)
            *ptr[j] = (T)v[j];  // whole block: this tile is its only writer
          else
            act |= 1u << j;
        }
      }
      atomic_max_entries<kPer>(ptr, v, act);
    }
    if (colw && kPairs && p.col_pair) {
      const int cc0 = 2 * threadIdx.x;        // columns cc, cc + 1 within the tile (WC = 512)
      const bool ok = cc0 < WC;               // threads past the tile's columns idle
      const int cc = ok ? cc0 : 0;
      const int ln = cc / E, q = (cc % E) / 2;  // lane and dword of s_col holding both
      uint32_t m = 0, t = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const uint4 o = s_col[w][ln];
        const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
        m = pk_max_u16(m, ov[q]);
        t |= s_touch[w][ln];
      }
      int mode[2] = {0, 0};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t cg = c0 + cc + h;
        // the block's first and last elements decide whether the piece holds it whole
        const int64_t gf = r0 * p.cols + cg, gl = (r0 + nrows - 1) * p.cols + cg;
        if (ok && cg < p.cols && ((t >> (2 * q + h)) & 1u)) mode[h] = (gf >= p.start && gl < p.end) ? 1 : 2;
      }
      if (mode[0] | mode[1])
        update_entry_pair(reinterpret_cast<uint32_t*>(static_cast<T*>(p.amax_col) + band * p.ld_ac +
                                                      c0 + cc),
                          m, mode[0], mode[1]);
    } else if (colw) {
      constexpr int kPer = WC >= kT ? WC / kT : 1;  // columns per thread (2 or 1 with 256 threads)
      T* ptr[kPer];
      uint32_t v[kPer], act = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int cc0 = threadIdx.x + j * kT;  // column within the tile
        const bool ok = cc0 < WC;              // threads past the tile's columns idle
        const int cc = ok ? cc0 : 0;
        const int ln = cc / E, e = cc % E;
        uint32_t m = 0, t = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const uint4 o = s_col[w][ln];
          const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
          m = umax(m, col_entry<T>(ov, e));
          t |= s_touch[w][ln];
        }
        ptr[j] = static_cast<T*>(p.amax_col) + band * p.ld_ac + c0 + cc;
        v[j] = m;
        // the block's first and last elements decide whether the piece holds it whole
        const int64_t gf = r0 * p.cols + c0 + cc, gl = (r0 + nrows - 1) * p.cols + c0 + cc;
        if (ok && c0 + cc < p.cols && ((t >> e) & 1u)) {
          if (gf >= p.start && gl < p.end)
            *ptr[j] = (T)m;
          else
            act |= 1u << j;
        }
      }
      atomic_max_entries<kPer>(ptr, v, act);
    }
  }
}

// ------------------------------------------------------------------ partial cast, vector path

// E4M3 bytes of one chunk with one exponent shift for all elements (row-wise) or one per
// element (column-wise), packed little-endian into E/4 dwords.
template <typename T, bool kPre>
__device__ __forceinline__ void quantize_chunk(const uint32_t (&d)[4], const int* shift,
                                               bool per_elem, uint32_t* out) {
  constexpr int E = Chunk<T>::E;
#pragma unroll
  for (int q = 0; q < E / 4; ++q) {
    float x[4];
    int s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      x[t] = work_value<T, kPre>(chunk_elem<T>(d, 4 * q + t));
      s[t] = per_elem ? shift[4 * q + t] : shift[0];
    }
    uint32_t w = cvt2<false>(x[0], x[1], s[0], s[1], 0);
    out[q] = cvt2<true>(x[2], x[3], s[2], s[3], w);
  }
}

// E output bytes of a chunk at p (4-byte aligned).  Where every output row of the piece starts
// on a 64-byte boundary (kNT), a wave's row of stores covers whole 64-byte pieces of its lines
// and streams out with non-temporal stores.  Otherwise the ends of each row segment share
// 64-byte pieces with the neighbouring workgroups' segments, and ordinary stores, which the L2
// holds and merges, cost less: 16384x6144 outputs 4 bytes off a line took the FP32 cast 152 us
// with streaming stores and 118 us with ordinary ones (102 us aligned; 112 us with streaming
// stores 64 bytes off a line, 118 us with ordinary ones).
// The two kinds must stay apart where a branch selects between them: merged into one store,
// the streaming hint is dropped.  So the ordinary store sits between two empty asm statements,
// compiler-only memory barriers that emit no instruction.
template <int E, bool kNT>
__device__ __forceinline__ void store_chunk(uint8_t* p, const uint32_t* q) {
  if constexpr (kNT) {
    if constexpr (E == 8)
      __builtin_nontemporal_store(v2u{q[0], q[1]}, reinterpret_cast<v2u*>(p));
    else
      __builtin_nontemporal_store(q[0], reinterpret_cast<uint32_t*>(p));
  } else {
    asm volatile("" ::: "memory");
    if constexpr (E == 8)
      *reinterpret_cast<v2u*>(p) = v2u{q[0], q[1]};
    else
      *reinterpret_cast<uint32_t*>(p) = q[0];
    asm volatile("" ::: "memory");
  }
}

// The same with the choice made at run time, one chunk at a time: the general and edge tiles
// of the cast.  The common cast tile takes only outputs whose rows start on 64-byte boundaries
// and streams; the single-pass quantize always streams.
template <int E>
__device__ __forceinline__ void store_bytes(uint8_t* p, const uint32_t* q, bool nt) {
  if (nt)
    store_chunk<E, true>(p, q);
  else
    store_chunk<E, false>(p, q);
}

template <int E>
__device__ __forceinline__ void store_masked(uint8_t* p, const uint32_t* q, uint32_t mask) {
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((mask >> e) & 1u) p[e] = (uint8_t)(q[e >> 2] >> ((e & 3) * 8));
}

// Bytes [lo, hi) of the word w into the dword at the 4-byte-aligned address a, with at most
// one byte store and one 2-byte store (lo == hi: nothing).  Used for the partial dwords at the
// two ends of a row segment whose outputs are not dword aligned, where the dword's other
// bytes belong to a neighbouring segment; every range that occurs is [mo, 4) or [0, mo).
__device__ __forceinline__ void store_partial(uint8_t* a, uint32_t w, int lo, int hi) {
  const int len = hi - lo;
  if (len & 1) {
    const int b = (lo & 1) ? lo : hi - 1;
    a[b] = (uint8_t)(w >> (8 * b));
  }
  if (len >= 2) {
    const int h = (lo & 1) ? lo + 1 : lo;
    *reinterpret_cast<uint16_t*>(a + h) = (uint16_t)(w >> (8 * h));
  }
}

// Chunk outputs at p, mo = p mod 4 != 0 (fragment-relative outputs not dword aligned); the
// lanes of a row segment hold consecutive chunks, `first` the segment's first lane and `last`
// its last.  Each lane writes the dword-aligned window [p - mo, p - mo + E): the last mo bytes
// of the lane to its left and its own first E - mo bytes.  The first lane's window would start
// with another segment's bytes: with E = 8 it writes [p - mo + 4, p - mo + 12) instead, its own
// bytes there followed by the next lane's first 4 - mo (the same bytes that lane writes), so
// one 8-byte store instruction serves every lane.  What is left are the partial dwords at the
// segment's two ends, the first lane's leading 4 - mo bytes and the last lane's trailing mo
// bytes, which share one byte and one 2-byte store instruction.  Neighbour words move by DPP
// wave shifts, so every lane of the wave must call this.
template <int E>
__device__ __forceinline__ void store_window(uint8_t* p, const uint32_t* q, int mo, bool valid,
                                             bool first, bool last) {
  uint32_t prev[E / 4];
#pragma unroll
  for (int j = 0; j < E / 4; ++j)  // wave_shr:1 (DPP 0x138): lane l reads lane l - 1
    prev[j] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q[j], 0x138, 0xF, 0xF, false);
  // wave_shl:1 (DPP 0x130): lane l reads lane l + 1
  const uint32_t next0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q[0], 0x130, 0xF, 0xF, false);
  if (!valid) return;
  const int sh = 8 * mo;
  uint8_t* a = p - mo;  // dword aligned
  uint32_t head, tail;  // the partial dwords' words: [mo, 4) of head at a, [0, mo) of tail
  if constexpr (E == 8) {
    const uint64_t own = ((uint64_t)q[1] << 32) | q[0];
    if (!first) {
      const uint64_t pv = ((uint64_t)prev[1] << 32) | prev[0];
      const uint64_t win = (own << sh) | (pv >> (64 - sh));
      __builtin_nontemporal_store(v2u{(uint32_t)win, (uint32_t)(win >> 32)},
                                  reinterpret_cast<v2u*>(a));
    } else if (!last) {
      const uint64_t win = (own >> (32 - sh)) | ((uint64_t)next0 << (32 + sh));
      __builtin_nontemporal_store(v2u{(uint32_t)win, (uint32_t)(win >> 32)},
                                  reinterpret_cast<v2u*>(a + 4));
    } else {
      __builtin_nontemporal_store((uint32_t)(own >> (32 - sh)),
                                  reinterpret_cast<uint32_t*>(a + 4));
    }
    head = (uint32_t)(own << sh);
    tail = (uint32_t)(own >> (64 - sh));
  } else {
    if (!first)
      __builtin_nontemporal_store((q[0] << sh) | (prev[0] >> (32 - sh)),
                                  reinterpret_cast<uint32_t*>(a));
    head = q[0] << sh;
    tail = q[0] >> (32 - sh);
  }
  // one byte and one 2-byte store instruction for the first lane's head and the last lane's
  // tail; a lone lane that is both writes its tail after
  int lo = 0, hi = 0;
  uint8_t* pa = a;
  uint32_t pw = head;
  if (first) {
    lo = mo;
    hi = 4;
  } else if (last) {
    hi = mo;
    pa = a + E;
    pw = tail;
  }
  store_partial(pa, pw, lo, hi);
  if (first && last) store_partial(a + E, tail, 0, mo);
}

// Fused scales: the E8M0 bytes of the lane's E column-wise blocks, from their amax entries.
template <typename T>
__device__ __forceinline__ void col_scales(const TileArgs& p, int64_t band, int64_t c,
                                           uint8_t (&s)[Chunk<T>::E]) {
  constexpr int E = Chunk<T>::E;
  const T* a = static_cast<const T*>(p.amax_col) + band * p.ld_ac + c;
  if (p.col_vec) {
    uint32_t d[4];
    load16(a, d);
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = e8m0_of<T>(chunk_elem<T>(d, e));
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = e8m0_of<T>(a[e]);
  }
}

// E scale bytes at p; bit e of mask selects byte e.  Whole dword-aligned runs go out as one
// store.
template <int E>
__device__ __forceinline__ void store_scale_bytes(uint8_t* p, const uint8_t (&s)[E],
                                                  uint32_t mask) {
  if (mask == (1u << E) - 1 && (reinterpret_cast<uintptr_t>(p) & 3) == 0) {
    uint32_t w[E / 4];
#pragma unroll
    for (int j = 0; j < E / 4; ++j)
      w[j] = s[4 * j] | (s[4 * j + 1] << 8) | (s[4 * j + 2] << 16) | ((uint32_t)s[4 * j + 3] << 24);
    if constexpr (E == 8)
      *reinterpret_cast<v2u*>(p) = v2u{w[0], w[1]};
    else
      *reinterpret_cast<uint32_t*>(p) = w[0];
    return;
  }
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((mask >> e) & 1u) p[e] = s[e];
}

// Fused scales: the amax entry of row-wise block (r, c / 32).
template <typename T>
__device__ __forceinline__ uint32_t row_amax(const TileArgs& p, int64_t r, int64_t c) {
  return static_cast<const T*>(p.amax_row)[r * p.ld_ar + (c >> 5)];
}

// Fused scales: wave 0 writes the scale bytes of the lane's column-wise blocks that the
// fragment touches (all of them in an interior tile).  Called after the tile's loads.
template <typename T>
__device__ __forceinline__ void store_col_scales(const TileArgs& p, int64_t band, int64_t c,
                                                 int nrows, bool interior,
                                                 const uint8_t (&sb)[Chunk<T>::E]) {
  constexpr int E = Chunk<T>::E;
  uint32_t m = (1u << E) - 1;
  if (!interior) {
    const Corners f = corners_of(p);
    const int64_t r0 = band * kBlockLen;
    m = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (col_block_touched(f, r0, r0 + nrows - 1, c + e)) m |= 1u << e;
  }
  store_scale_bytes<E>(p.scale_col + band * p.ld_sc + c, sb, m);
}

// Not fused: the column-wise scale bytes of the lane's E columns, as loaded: one vector when
// scale_col rows are aligned to E bytes (cw[0 .. E/4) hold the packed bytes), else one load
// per byte (cw[e]).  col_shifts_of turns them into exponent shifts once they have arrived.
template <typename T>
__device__ __forceinline__ void col_scale_raw(const TileArgs& p, int64_t band, int64_t c,
                                              uint32_t (&cw)[Chunk<T>::E]) {
  constexpr int E = Chunk<T>::E;
  const uint8_t* sc = p.scale_col + band * p.ld_sc + c;
#pragma unroll
  for (int e = 0; e < E; ++e) cw[e] = 0;
  if (p.sc_vec) {
    if constexpr (E == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(sc);
      cw[0] = v.x;
      cw[1] = v.y;
    } else {
      cw[0] = *reinterpret_cast<const uint32_t*>(sc);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) cw[e] = sc[e];
  }
}

template <typename T>
__device__ __forceinline__ void col_shifts_of(const TileArgs& p, const uint32_t (&cw)[Chunk<T>::E],
                                              int (&cshift)[Chunk<T>::E]) {
  constexpr int E = Chunk<T>::E;
#pragma unroll
  for (int e = 0; e < E; ++e)
    cshift[e] = 127 - (int)(p.sc_vec ? (cw[e >> 2] >> (8 * (e & 3))) & 0xFFu : cw[e]);
}

// Tiles a fragment boundary or the short last band cuts (kEdge: masked loads and stores), and
// interior tiles whose outputs are not dword aligned (window stores).  The common tile
// (interior, dword-aligned outputs) takes its own straight-line block in cast_vec_kernel.  The
// two kinds are separate instances, so that no edge tile's code follows a join with loads that
// an interior tile would have in flight (the compiler would wait for those too).
template <typename T, bool kCol, bool kPre, bool kFuse, bool kEdge, int kSplit = 1>
__device__ __forceinline__ void cast_tile_general(
    const TileArgs& p, int64_t band, int64_t r0, int64_t c0, int64_t c, int i0, int nrows,
    int (&cshift)[Chunk<T>::E], bool colw) {
  constexpr bool interior = !kEdge;
  constexpr int E = Chunk<T>::E;
  constexpr int WC = kWaveSize * E;
  constexpr int RW = kRowsPerWave / kSplit;
  constexpr uint32_t kFull = (1u << E) - 1;
  const int lane = threadIdx.x & (kWaveSize - 1);
  const bool cvalid = c < p.cols;
  const int64_t cend = min<int64_t>(c0 + WC, p.cols);
  const bool first = lane == 0, last = c + E == cend;
  const T* src = static_cast<const T*>(p.input) + ((r0 + i0) * p.cols + c - p.start);
  const uint8_t* srow = p.scale_row + (r0 + i0) * p.ld_sr + (c >> 5);
  const int64_t o0 = (r0 + i0) * p.cols + c - p.start;
  uint32_t d[RW][4], em[RW];
  int rshift[RW];
  // Every load of the tile goes out before any value is used: the input rows (interior tiles
  // here; edge tiles, once classified, after the scale loads: the assembly in load_rows_masked
  // then waits for them all), the row-wise scale bytes or (fused) amax entries, and (not
  // fused) the column-wise scale bytes.  The scale loads are unconditional, a lane that needs
  // none reading the tile's first one (dropped): a load under a per-lane condition makes the
  // compiler wait for it where the branches join.
  RowClass<RW> rc;
  if constexpr (interior) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      d[i][0] = d[i][1] = d[i][2] = d[i][3] = 0;
      em[i] = cvalid ? kFull : 0u;
    }
    if (cvalid) load_rows<T, RW>(src, p.cols, p.in_shift2, RW, d, c0 + WC <= p.cols);
  } else {
    rc = classify_rows<T, RW>(p, r0 + i0, nrows - i0, c, cvalid);
#pragma unroll
    for (int i = 0; i < RW; ++i) em[i] = rc.em[i];
    // fused: the rows first, which keeps the column-wise amax entries' registers free sooner
    if constexpr (kFuse) load_rows_masked<T, RW>(p, src, r0 + i0, c, rc, d);
  }
  uint32_t rl[RW];  // row-wise scale bytes or (fused) amax entries, as loaded
  bool wr[RW];      // (fused) the lane writes row i's scale byte
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    if constexpr (kFuse) {
      // the first lane of each row-wise block writes the scale of a block the fragment touches
      wr[i] = (lane & (kBlockLen / E - 1)) == 0 && cvalid && i < nrows - i0 &&
              (interior || row_block_touched(p, r0 + i0 + i, c));
      const bool need = em[i] || wr[i];
      rl[i] = row_amax<T>(p, need ? r0 + i0 + i : r0, need ? c : c0);
    } else {
      wr[i] = false;
      rl[i] = em[i] ? srow[i * p.ld_sr] : p.scale_row[r0 * p.ld_sr + (c0 >> 5)];
    }
  }
  uint32_t cw[E];  // (not fused) the lane's column-wise scale bytes, as loaded
  if (!kFuse && colw) col_scale_raw<T>(p, band, cvalid ? c : c0, cw);
  if constexpr (!kFuse && kEdge) load_rows_masked<T, RW>(p, src, r0 + i0, c, rc, d);
  if constexpr (kFuse) {
    // every amax entry was loaded before the first store, so no load waits on one
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const uint8_t sb = e8m0_of<T>((em[i] || wr[i]) ? rl[i] : 0u);
      rshift[i] = 127 - (int)sb;
      if (wr[i]) p.scale_row[(r0 + i0 + i) * p.ld_sr + (c >> 5)] = sb;
    }
  } else {
    if (colw && cvalid) col_shifts_of<T>(p, cw, cshift);
#pragma unroll
    for (int i = 0; i < RW; ++i) rshift[i] = em[i] ? 127 - (int)rl[i] : 0;
  }
  if constexpr (interior) {  // outputs not dword aligned: window stores (every lane takes part)
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      uint32_t q[E / 4];
      quantize_chunk<T, kPre>(d[i], &rshift[i], false, q);
      if (p.mo_row)
        store_window<E>(p.data_row + o0 + i * p.cols, q, p.mo_row, cvalid, first, last);
      else if (cvalid)
        store_bytes<E>(p.data_row + o0 + i * p.cols, q, p.nt_row);
    }
    if (colw) {
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        uint32_t q[E / 4];
        quantize_chunk<T, kPre>(d[i], cshift, true, q);
        if (p.mo_col)
          store_window<E>(p.data_col + o0 + i * p.cols, q, p.mo_col, cvalid, first, last);
        else if (cvalid)
          store_bytes<E>(p.data_col + o0 + i * p.cols, q, p.nt_col);
      }
    }
  } else {
    // edge tile: whole chunks store whole when the outputs are dword aligned, else byte by byte
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if (!em[i]) continue;
      const int64_t o = o0 + i * p.cols;
      uint32_t q[E / 4];
      quantize_chunk<T, kPre>(d[i], &rshift[i], false, q);
      if (em[i] == kFull && p.mo_row == 0)
        store_bytes<E>(p.data_row + o, q, p.nt_row);
      else
        store_masked<E>(p.data_row + o, q, em[i]);
      if (colw) {
        quantize_chunk<T, kPre>(d[i], cshift, true, q);
        if (em[i] == kFull && p.mo_col == 0)
          store_bytes<E>(p.data_col + o, q, p.nt_col);
        else
          store_masked<E>(p.data_col + o, q, em[i]);
      }
    }
  }
}

// Same tiling as the amax: a workgroup per (band, 64*E columns), wave w casts rows 8w..8w+7
// with all loads in flight.  kGuard as for the amax (not fused): the column-wise work
// follows a run-time test of data_col.  kScaleFirst (not fused): the common tile loads its
// scale bytes before its input rows (see there).  kSplit (launches too small to fill the
// GPU): a workgroup takes 32 / kSplit rows of a band, wave w rows (8 / kSplit) w ... , so each
// wave's serial work, an edge tile's above all, is kSplit times shorter; tile t of a piece is
// then (sub-band t / ntc, column tile t % ntc).  kOne as for the amax.
template <typename T, bool kCol, bool kPre, bool kFuse, int kOcc, bool kGuard = false,
          bool kScaleFirst = false, int kSplit = 1, bool kOne = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kOcc))) void cast_vec_kernel(GroupArgs ga) {
  constexpr int E = Chunk<T>::E;
  constexpr int WC = kWaveSize * E;
  constexpr int RW = kRowsPerWave / kSplit;
  constexpr int kTileRows = kBlockLen / kSplit;
  static_assert(kSplit == 1 || !kScaleFirst, "split tiles: small launches");

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = threadIdx.x >> 6;
  if constexpr (!kOne) pin_header(ga);
  const uint32_t lt = xcd_remap(blockIdx.x, gridDim.x);  // tile of the launch
  const int k = kOne ? 0 : piece_of(ga, lt);  // a launch of one piece: piece 0
  const TileArgs& p = ga.piece[k];
  pin_cast_fields(ga, k);
  const int64_t tile = (int64_t)(lt - ga.first[k]) + p.tile0;
  if (tile >= p.ntiles) return;  // uniform over the workgroup
  const uint32_t t32 = (uint32_t)tile, n32 = (uint32_t)p.ntc, bq = t32 / n32;
  const int64_t band = p.band0 + bq / kSplit;
  const int64_t c0 = (int64_t)(t32 - bq * n32) * WC;
  const int64_t c = c0 + lane * E;
  const int64_t r0 = band * kBlockLen + (int64_t)(bq % kSplit) * kTileRows;  // the tile's first row
  if (kSplit > 1 && r0 >= p.rows) return;  // a short last band's missing rows (uniform)
  // (fused) the band's column-wise scale bytes are written once, by its first sub-tile, which
  // tests every column block against the fragment over all the band's rows
  const bool col_writer = kSplit == 1 || bq % kSplit == 0;
  const int band_rows = (int)min<int64_t>(kBlockLen, p.rows - band * kBlockLen);
  const bool cvalid = c < p.cols;
  const int nrows = (int)min<int64_t>(kTileRows, p.rows - r0);
  const int i0 = wave * RW;
  const int64_t tile_first = r0 * p.cols + c0;
  const int64_t tile_end = (r0 + nrows - 1) * p.cols + min<int64_t>(c0 + WC, p.cols);
  // (with && rather than &: the fields are pinned already, and & slowed the edge tiles by
  // 0.3 µs in a call of one round)
  const bool interior = nrows == kTileRows && tile_first >= p.start && tile_end <= p.end;
  static_assert(!(kGuard && kFuse), "the runtime-guard ablation covers the plain cast");
  const bool colw = kCol && (!kGuard || p.data_col != nullptr);  // column-wise output

  // Column-wise shifts and (fused) scale bytes.  Fused: from the amax entries, here, before
  // the tile's loads (measured faster than with them); otherwise from the scale bytes, loaded
  // after the tile's other loads.
  int cshift[E];
  uint8_t csb[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    cshift[e] = 0;
    csb[e] = 0;
  }
  if constexpr (kCol && kFuse) {
    if (cvalid) {
      col_scales<T>(p, band, c, csb);
#pragma unroll
      for (int e = 0; e < E; ++e) cshift[e] = 127 - (int)csb[e];
    }
  }

  // the common tile: interior, outputs whose rows start on 64-byte boundaries (streaming stores)
  // and (not fused) column-wise scale bytes that move as one vector; straight-line code
  if (interior && p.nt_row && (!colw || p.nt_col) && (!colw || kFuse || p.sc_vec)) {
    if (!cvalid) return;
    const T* src = static_cast<const T*>(p.input) + ((r0 + i0) * p.cols + c - p.start);
    const uint8_t* srow = p.scale_row + (r0 + i0) * p.ld_sr + (c >> 5);
    const int64_t o0 = (r0 + i0) * p.cols + c - p.start;
    uint32_t d[RW][4];
    int rshift[RW];
    // Every load of the tile goes out before any value is used, and before the first store
    // (which the compiler cannot move a load past): the input rows and the row-wise amax
    // entries (fused) or scale bytes and (not fused) the column-wise scale bytes.  Loads
    // complete in order, so with the input first a wave waits for every row before it casts
    // the first (its scale bytes come last), and the compiler spreads the scale loads between
    // waits for rows.  kScaleFirst puts the scale bytes first: each row is cast once it
    // arrives, which pays where workgroups follow one another on a CU (the bidirectional BF16
    // cast of 16384x6144, 6144 tiles: 71.3 -> 69.9 us); in a launch of one round (a quarter of
    // it), where the scale loads only delay the input's, for FP32 and for the row-only BF16
    // cast it cost about 1%.
    static_assert(!(kScaleFirst && kFuse), "the fused cast loads amax entries instead");
    uint32_t cw[2] = {0, 0};
    uint32_t rl[RW];
    auto load_scales = [&] {
#pragma unroll
      for (int i = 0; i < RW; ++i)
        rl[i] = kFuse ? row_amax<T>(p, r0 + i0 + i, c) : (uint32_t)srow[i * p.ld_sr];
      if (colw && !kFuse) {
        if constexpr (E == 8) {
          const uint2 v = *reinterpret_cast<const uint2*>(p.scale_col + band * p.ld_sc + c);
          cw[0] = v.x;
          cw[1] = v.y;
        } else {
          cw[0] = *reinterpret_cast<const uint32_t*>(p.scale_col + band * p.ld_sc + c);
        }
      }
    };
    if constexpr (kScaleFirst) load_scales();
    load_rows<T, RW>(src, p.cols, p.in_shift2, RW, d, c0 + WC <= p.cols);
    if constexpr (!kScaleFirst) load_scales();
    if (colw && !kFuse) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        csb[e] = (uint8_t)(cw[e >> 2] >> (8 * (e & 3)));
        cshift[e] = 127 - (int)csb[e];
      }
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if constexpr (kFuse) {
        const uint8_t sb = e8m0_of<T>(rl[i]);
        rshift[i] = 127 - (int)sb;
        if ((lane & (kBlockLen / E - 1)) == 0) p.scale_row[(r0 + i0 + i) * p.ld_sr + (c >> 5)] = sb;
      } else {
        rshift[i] = 127 - (int)rl[i];
      }
    }
    // all row-wise stores, then all column-wise ones: each output gets one run of stores
    // (interleaving the two directions measured 1.4% slower)
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      uint32_t q[E / 4];
      quantize_chunk<T, kPre>(d[i], &rshift[i], false, q);
      store_chunk<E, true>(p.data_row + o0 + i * p.cols, q);
    }
    if (colw) {
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        uint32_t q[E / 4];
        quantize_chunk<T, kPre>(d[i], cshift, true, q);
        store_chunk<E, true>(p.data_col + o0 + i * p.cols, q);
      }
    }
    if constexpr (kFuse && kCol) {
      if (wave == 0 && col_writer) store_col_scales<T>(p, band, c, band_rows, kSplit == 1, csb);
    }
    return;
  }
  if (interior)
    cast_tile_general<T, kCol, kPre, kFuse, false, kSplit>(p, band, r0, c0, c, i0, nrows, cshift, colw);
  else
    cast_tile_general<T, kCol, kPre, kFuse, true, kSplit>(p, band, r0, c0, c, i0, nrows, cshift, colw);
  if constexpr (kFuse && kCol) {
    if (wave == 0 && cvalid && col_writer)
      store_col_scales<T>(p, band, c, band_rows, kSplit == 1 && interior, csb);
  }
}

// ------------------------------------------------------------------ partial cast, line-owned tiles

// Fragment-sized outputs (each rank's E4M3 bytes in buffers of the fragment's own size) put
// data - start at an arbitrary byte offset, so the standard tiles' output row segments begin
// and end inside 128-byte lines that two workgroups write at different times.  These tiles
// are laid out in output-address space instead.  With delta = (-(data_row - start)) mod 128
// (kLineBytes) and cols a multiple of 128, tile (virtual band B, column tile j) covers, for
// each virtual row v of [32 B, 32 B + 32), the contiguous flat range
//   [v cols + delta + 64 E j,  v cols + delta + min(64 E (j + 1), cols)),
// which starts on a line of the row-wise output.  A virtual row holds columns delta .. cols-1
// of row v and then columns 0 .. delta-1 of row v + 1, so the tiles still cover every element
// once, every workgroup writes whole lines of both outputs (the column-wise output has the
// same offset), and the input is streamed exactly as in the standard tiles: a virtual row is
// contiguous in memory.  The price is in the scale lookups: a lane's chunk can hold elements
// of two row-wise blocks or of two rows, so its row-wise scale comes per element from two
// scale bytes per row, and its column-wise scales from one or two byte windows of scale_col.
// The n (1 <= n <= 4 W) bytes at any byte address a, little-endian in W dwords (bytes past n
// are unspecified): the dwords that hold them, joined by byte funnel shifts.  Only dwords that
// hold one of the n bytes are read.
template <int W>
__device__ __forceinline__ void load_window(const uint8_t* a, int n, uint32_t (&w)[W]) {
  const uintptr_t ai = reinterpret_cast<uintptr_t>(a);
  global_cu32* d = global_cdword(ai);
  const int last = (int)(((ai + (uintptr_t)n - 1) >> 2) - (ai >> 2));  // last dword to read
  const int sh = (int)(ai & 3);
  uint32_t x[W + 1];
#pragma unroll
  for (int j = 0; j <= W; ++j) x[j] = d[j < last ? j : last];
#pragma unroll
  for (int j = 0; j < W; ++j) w[j] = __builtin_amdgcn_alignbyte(x[j + 1], x[j], sh);
}

// Column-wise scale bytes of a lane's E elements, packed little-endian: elements e < eC are
// column cA + e of band bandA, the others (a chunk that runs past the row's end) column
// e - eC of band bandB.  Issues its loads and uses them, so the caller calls it after the
// tile's input loads.  Kept packed (E / 4 registers), the bytes become shifts at each use.
template <int E>
__device__ __forceinline__ uint64_t lines_col_scales(const TileArgs& p, int64_t bandA,
                                                     int64_t bandB, int64_t cA, int eC) {
  constexpr int W = E / 4;
  uint32_t a[W], b[W];
  load_window<W>(p.scale_col + bandA * p.ld_sc + cA, eC, a);
  load_window<W>(p.scale_col + bandB * p.ld_sc, eC < E ? E - eC : 1, b);
  uint64_t av = a[0], bv = b[0];
  if constexpr (W == 2) {
    av |= (uint64_t)a[1] << 32;
    bv |= (uint64_t)b[1] << 32;
  }
  bv = eC < E ? bv << (8 * eC) : 0;  // byte e of bv: column e - eC of band bandB
  const uint64_t lo = eC < 8 ? (uint64_t(1) << (8 * eC)) - 1 : ~uint64_t(0);  // bytes e < eC
  return (av & lo) | (bv & ~lo);
}

// Exponent shifts from packed scale bytes.
template <int E>
__device__ __forceinline__ void unpack_shifts(uint64_t packed, int (&sh)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) sh[e] = 127 - (int)((packed >> (8 * e)) & 0xFFu);
}

template <typename T, bool kCol, bool kPre, int kOcc>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kOcc))) void cast_lines_kernel(GroupArgs ga) {
  constexpr int E = Chunk<T>::E;
  constexpr int WC = kWaveSize * E;
  constexpr int RW = kRowsPerWave;
  constexpr uint32_t kFull = (1u << E) - 1;

  const int lane = threadIdx.x & (kWaveSize - 1);
  // uniform over the wave: row addresses stay in scalar registers, a lane adds its offset
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  pin_header(ga);
  const uint32_t lt = xcd_remap(blockIdx.x, gridDim.x);  // tile of the launch
  const int k = piece_of(ga, lt);
  const TileArgs& p = ga.piece[k];
  pin_tile_fields(ga, k);
  const int64_t tile = (int64_t)(lt - ga.first[k]) + p.tile0;
  if (tile >= p.ntiles) return;  // uniform over the workgroup
  const uint32_t t32 = (uint32_t)tile, n32 = (uint32_t)p.ntc, bq = t32 / n32;
  const int64_t vband = p.band0 + bq;  // virtual band; -1 holds row 0's first delta columns
  const int64_t u0 = (int64_t)(t32 - bq * n32) * WC;
  const bool cvalid = u0 + lane * E < p.cols;
  const int64_t u = cvalid ? u0 + lane * E : 0;  // the lane's virtual column
  const int64_t v0 = vband * kBlockLen;
  const int i0 = wave * RW;
  const int64_t cu = u + p.shift;
  const int64_t tile_first = v0 * p.cols + p.shift + u0;
  const int64_t tile_last = (v0 + kBlockLen - 1) * p.cols + p.shift + min<int64_t>(u0 + WC, p.cols) - 1;
  const bool interior = (tile_first >= p.start) & (tile_last < p.end);
  const bool last_tc = u0 + WC >= p.cols;  // the column tile whose chunks reach the next row

  // Where the lane's chunk lies, the same for every row: wholly in the next row (wrap), across
  // the row's end (strad), or inside row v, where it may still cross a row-wise block boundary.
  const bool wrap = cu >= p.cols;
  const int64_t cA = wrap ? cu - p.cols : cu;  // real column of the chunk's first element
  const bool strad = !wrap && cu + E > p.cols;
  const int eC = strad ? (int)(p.cols - cA) : E;  // elements in the first element's row
  const int eS = strad ? eC : min(E, kBlockLen - (int)(cA & (kBlockLen - 1)));  // ... and block
  const int offA = wrap ? 1 : 0, offB = (wrap || strad) ? 1 : 0;  // rows after v
  const int64_t kA = cA >> 5, kB = strad ? 0 : (cA + E - 1) >> 5;  // the two row-wise blocks
  const int64_t last_row = p.rows - 1, last_band = (p.rows - 1) / kBlockLen;
  auto clamp_row = [&](int64_t r) { return r < 0 ? 0 : (r > last_row ? last_row : r); };
  auto clamp_band = [&](int64_t b) { return b < 0 ? 0 : (b > last_band ? last_band : b); };

  const T* src = static_cast<const T*>(p.input) + ((v0 + i0) * p.cols + cu - p.start);
  const int64_t o0 = (v0 + i0) * p.cols + cu - p.start;
  uint32_t d[RW][4], em[RW];
  if (interior) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      d[i][0] = d[i][1] = d[i][2] = d[i][3] = 0;
      em[i] = cvalid ? kFull : 0u;
    }
    if (cvalid) load_rows<T, RW>(src, p.cols, p.in_shift2, RW, d, u0 + WC <= p.cols);
  } else {
    const RowClass<RW> rc = classify_rows<T, RW>(p, v0 + i0, RW, cu, cvalid);
#pragma unroll
    for (int i = 0; i < RW; ++i) em[i] = rc.em[i];
    load_rows_masked<T, RW>(p, src, v0 + i0, cu, rc, d);
  }
  // The two row-wise scale bytes of every row.  In an interior tile every row exists: each is
  // at a fixed lane offset from the row's first scale byte, a scalar address (the host keeps
  // the offsets below 2^31).  Edge tiles clamp the rows (rows outside the weight hold no
  // element of the fragment).
  uint32_t sa[RW], sb[RW];
  if (interior) {
    const uint32_t oa = (uint32_t)(offA * p.ld_sr + kA), ob = (uint32_t)(offB * p.ld_sr + kB);
    const uint8_t* rb = p.scale_row + (v0 + i0) * p.ld_sr;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      sa[i] = rb[oa];
      sb[i] = rb[ob];
      rb += p.ld_sr;
    }
  } else {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      sa[i] = p.scale_row[clamp_row(v0 + i0 + i + offA) * p.ld_sr + kA];
      sb[i] = p.scale_row[clamp_row(v0 + i0 + i + offB) * p.ld_sr + kB];
    }
  }
  // column-wise scale bytes: every row of the tile uses band B, except the next-row elements
  // of the last virtual row (wave 3, row 7), which belong to band B + 1
  uint64_t csp = 0, csp7 = 0;
  if constexpr (kCol) {
    const int64_t bm = clamp_band(vband);
    csp = lines_col_scales<E>(p, bm, bm, cA, eC);
    csp7 = csp;
    if (wave == kWavesPerGroup - 1 && last_tc)
      csp7 = lines_col_scales<E>(p, clamp_band(vband + offA), clamp_band(vband + offB), cA, eC);
  }

#pragma unroll
  for (int i = 0; i < RW; ++i) {
    if (!em[i]) continue;
    int rs[E];
#pragma unroll
    for (int e = 0; e < E; ++e) rs[e] = 127 - (int)(e < eS ? sa[i] : sb[i]);
    uint32_t q[E / 4];
    quantize_chunk<T, kPre>(d[i], rs, true, q);
    uint8_t* out = p.data_row + o0 + i * p.cols;
    if (interior)
      store_chunk<E, true>(out, q);
    else if (em[i] == kFull)
      store_chunk<E, false>(out, q);
    else
      store_masked<E>(out, q, em[i]);
  }
  if constexpr (kCol) {
    int cs[E];
    unpack_shifts<E>(csp, cs);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if (i == RW - 1 && wave == kWavesPerGroup - 1 && last_tc) unpack_shifts<E>(csp7, cs);
      if (!em[i]) continue;
      uint32_t q[E / 4];
      quantize_chunk<T, kPre>(d[i], cs, true, q);
      uint8_t* out = p.data_col + o0 + i * p.cols;
      if (interior)
        store_chunk<E, true>(out, q);
      else if (em[i] == kFull)
        store_chunk<E, false>(out, q);
      else
        store_masked<E>(out, q, em[i]);
    }
  }
}

// ------------------------------------------------------------------ single-pass quantize

// A fragment made of whole 32-row bands holds every block it touches entirely, so its block
// amax are final without any combine: one pass reads each tile once, keeps it in registers,
// reduces the row-wise blocks with DPP and the column-wise blocks over the four waves in LDS,
// and writes the amax (when requested), the E8M0 scales and the E4M3 data.  All loads are
// issued before the first store.  kWaves and kOne as for the amax.
template <typename T, bool kCol, bool kPre, int kOcc, int kWaves = kWavesPerGroup,
          bool kOne = false>
__global__ __launch_bounds__(kWaveSize * kWaves)
__attribute__((amdgpu_waves_per_eu(kOcc))) void quantize_vec_kernel(GroupArgs ga) {
  constexpr int E = Chunk<T>::E;
  constexpr int LB = kBlockLen / E;
  constexpr int WC = kWaveSize * E;
  constexpr int RW = kBlockLen / kWaves;  // rows of the band per wave (8; 4 with 8 waves)
  __shared__ uint4 s_col[kWaves][kWaveSize];

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = threadIdx.x >> 6;
  if constexpr (!kOne) pin_header(ga);
  const uint32_t lt = xcd_remap(blockIdx.x, gridDim.x);  // tile of the launch
  const int k = kOne ? 0 : piece_of(ga, lt);  // a launch of one piece: piece 0
  const TileArgs& p = ga.piece[k];
  pin_tile_fields(ga, k);
  const int64_t tile = (int64_t)(lt - ga.first[k]) + p.tile0;
  if (tile >= p.ntiles) return;  // uniform over the workgroup
  const uint32_t t32 = (uint32_t)tile, n32 = (uint32_t)p.ntc, bq = t32 / n32;
  const int64_t band = p.band0 + bq;
  const int64_t c0 = (int64_t)(t32 - bq * n32) * WC;
  const int64_t c = c0 + lane * E;
  const int64_t r0 = band * kBlockLen;
  const bool cvalid = c < p.cols;
  const int nrows = (int)min<int64_t>(kBlockLen, p.rows - r0);
  const int i0 = wave * RW;
  const int nr = nrows - i0;  // rows of this wave inside the weight (uniform; may be <= 0)

  const T* src = static_cast<const T*>(p.input) + ((r0 + i0) * p.cols + c - p.start);
  uint32_t d[RW][4];
#pragma unroll
  for (int i = 0; i < RW; ++i) d[i][0] = d[i][1] = d[i][2] = d[i][3] = 0;
  if (cvalid) {
    if (nr >= RW)
      load_rows<T, RW>(src, p.cols, p.in_shift2, RW, d, c0 + WC <= p.cols);
    else
      load_rows<T, RW>(src, p.cols, p.in_shift2, nr, d, c0 + WC <= p.cols);
  }

  // amax: rows absent from a short last band, and lanes past the last column, hold zeros
  uint32_t col[4] = {0, 0, 0, 0};
  uint32_t rmax[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) rmax[i] = group_max<LB>(chunk_absmax<T, kCol, kPre>(d[i], col));
  if constexpr (kCol) {
    s_col[wave][lane] = make_uint4(col[0], col[1], col[2], col[3]);
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (w != wave) fold_col<T>(col, s_col[w][lane]);
  }

  // row-wise amax and scales: the first lane of each block writes them
  int rshift[RW];
  const bool writer = (lane % LB) == 0 && cvalid;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const uint8_t sb = e8m0_of<T>(rmax[i]);
    rshift[i] = 127 - (int)sb;
    if (writer && i < nr) {
      const int64_t r = r0 + i0 + i;
      p.scale_row[r * p.ld_sr + (c >> 5)] = sb;
      if (p.amax_row) static_cast<T*>(p.amax_row)[r * p.ld_ar + (c >> 5)] = (T)rmax[i];
    }
  }
  int cshift[E];
  uint8_t csb[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    csb[e] = kCol ? e8m0_of<T>(col_entry<T>(col, e)) : 0;
    cshift[e] = 127 - (int)csb[e];
  }

  // data: direct stores when the outputs are dword aligned, else window stores; all
  // row-wise stores first, then the column-wise ones
  const int64_t o0 = (r0 + i0) * p.cols + c - p.start;
  const int64_t cend = min<int64_t>(c0 + WC, p.cols);
  const bool first = lane == 0, last = c + E == cend;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const bool valid = cvalid && i < nr;
    uint32_t q[E / 4];
    quantize_chunk<T, kPre>(d[i], &rshift[i], false, q);
    if (p.mo_row)
      store_window<E>(p.data_row + o0 + i * p.cols, q, p.mo_row, valid, first, last);
    else if (valid)
      store_chunk<E, true>(p.data_row + o0 + i * p.cols, q);
  }
  if constexpr (kCol) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const bool valid = cvalid && i < nr;
      uint32_t q[E / 4];
      quantize_chunk<T, kPre>(d[i], cshift, true, q);
      if (p.mo_col)
        store_window<E>(p.data_col + o0 + i * p.cols, q, p.mo_col, valid, first, last);
      else if (valid)
        store_chunk<E, true>(p.data_col + o0 + i * p.cols, q);
    }
  }

  // column-wise amax and scales: wave 0 writes them
  if constexpr (kCol) {
    if (wave == 0 && cvalid) {
      store_scale_bytes<E>(p.scale_col + band * p.ld_sc + c, csb, (1u << E) - 1);
      if (p.amax_col) {
        T* ac = static_cast<T*>(p.amax_col) + band * p.ld_ac + c;
        if (p.col_vec) {
          *reinterpret_cast<uint4*>(ac) = make_uint4(col[0], col[1], col[2], col[3]);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) ac[e] = (T)col_entry<T>(col, e);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ element-wise path (any layout)

constexpr int kElemTileCols = kWaveSize;  // one lane per column

// One wave per tile of a 32-row band x 64 columns, one lane per column.  All 32 rows are
// loaded before anything is written.  Each row's two row-wise blocks are reduced over the
// half-waves and lane 2i + h keeps block h of row i, so the tile's 64 row-wise entries are
// merged at the end, one per lane, together with the lane's column-wise entry: no load of a
// row waits on the entry update of the row before it.  Row addresses and the fragment's
// bounds within each row are uniform over the wave (scalar registers); a lane adds only its
// column.
template <typename T, bool kCol, bool kPre>
__global__ __launch_bounds__(kThreads) void amax_elem_kernel(GroupArgs ga) {
  const int lane = threadIdx.x & (kWaveSize - 1);
  // the wave index is uniform over the wave: readfirstlane lets the compiler keep the tile's
  // indices and addresses in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  pin_header(ga);
  const uint32_t lt = xcd_remap(blockIdx.x, gridDim.x) * kWavesPerGroup + wave;
  const int k = piece_of(ga, lt);
  const TileArgs& p = ga.piece[k];
  pin_tile_fields(ga, k);
  const int64_t tile = (int64_t)(lt - ga.first[k]) + p.tile0;
  if (tile >= p.ntiles) return;
  const int64_t band = p.band0 + tile / p.ntc;
  const int64_t c0 = (tile % p.ntc) * kElemTileCols;
  const int64_t r0 = band * kBlockLen;
  const int ncols = (int)min<int64_t>(kElemTileCols, p.cols - c0);  // lanes with a column
  const int nrows = (int)min<int64_t>(kBlockLen, p.rows - r0);
  const T* in_base = static_cast<const T*>(p.input);
  uint32_t a[kBlockLen];
  uint32_t in = 0;  // bit i: element (r0 + i, c0 + lane) lies in the fragment
#pragma unroll
  for (int i = 0; i < kBlockLen; ++i) {
    const int64_t g0 = (r0 + i) * p.cols + c0;  // flat index of the row's lane 0
    const int lo = (int)max<int64_t>(0, min<int64_t>(kElemTileCols, p.start - g0));
    const int hi = i < nrows ? (int)max<int64_t>(0, min<int64_t>(ncols, p.end - g0)) : 0;
    const bool inside = lane >= lo && lane < hi;
    // every lane loads (lanes outside the fragment read its first element), so no load sits
    // in a branch that would wait for it
    const uint32_t v = load_raw(in_base, inside ? g0 - p.start + lane : 0, (int)sizeof(T));
    a[i] = inside ? abs_bits<T, kPre>(v) : 0u;
    in |= (uint32_t)inside << i;
  }
  const uint64_t valid = __ballot(lane < ncols);
  uint32_t cmax = 0, rv = 0;
  bool rin = false, rfull = false;
#pragma unroll
  for (int i = 0; i < kBlockLen; ++i) {
    if constexpr (kCol) cmax = umax(cmax, a[i]);
    const uint32_t m = half_wave_max(a[i]);
    const uint64_t inb = __ballot((in >> i) & 1u);
    if (lane == 2 * i) {
      rv = __builtin_amdgcn_readlane(m, 0);
      rin = (uint32_t)inb != 0;
      rfull = (uint32_t)inb == (uint32_t)valid;
    }
    if (lane == 2 * i + 1) {
      rv = __builtin_amdgcn_readlane(m, 32);
      rin = (uint32_t)(inb >> 32) != 0;
      rfull = (uint32_t)(inb >> 32) == (uint32_t)(valid >> 32);
    }
  }
  if (rin) write_entry<T>(p.amax_row, (r0 + (lane >> 1)) * p.ld_ar + (c0 >> 5) + (lane & 1), rv, rfull);
  if constexpr (kCol) {
    const uint32_t all = nrows == kBlockLen ? ~0u : (1u << nrows) - 1u;
    if (in != 0) write_entry<T>(p.amax_col, band * p.ld_ac + c0 + lane, cmax, in == all);
  }
}

// Same tiling.  Lane 2i + h fetches the scale (or, fused, the amax entry) of block h of row i
// and every lane its column's, then all 32 rows are loaded, and only then is anything
// written; each row's two block scales reach their half-waves by readlane.
template <typename T, bool kCol, bool kPre, bool kFuse>
__global__ __launch_bounds__(kThreads) void cast_elem_kernel(GroupArgs ga) {
  const int lane = threadIdx.x & (kWaveSize - 1);
  // the wave index is uniform over the wave: readfirstlane lets the compiler keep the tile's
  // indices and addresses in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  pin_header(ga);
  const uint32_t lt = xcd_remap(blockIdx.x, gridDim.x) * kWavesPerGroup + wave;
  const int k = piece_of(ga, lt);
  const TileArgs& p = ga.piece[k];
  pin_tile_fields(ga, k);
  const int64_t tile = (int64_t)(lt - ga.first[k]) + p.tile0;
  if (tile >= p.ntiles) return;
  const int64_t band = p.band0 + tile / p.ntc;
  const int64_t c0 = (tile % p.ntc) * kElemTileCols;
  const int64_t r0 = band * kBlockLen;
  const int ncols = (int)min<int64_t>(kElemTileCols, p.cols - c0);
  const int nrows = (int)min<int64_t>(kBlockLen, p.rows - r0);
  const bool cvalid = lane < ncols;
  const int64_t rb = r0 + (lane >> 1);                 // the lane's row-wise block: row rb,
  const int64_t cb = c0 + kBlockLen * (lane & 1);      // columns from cb
  const bool bvalid = (lane >> 1) < nrows && cb < p.cols;
  // unconditional loads (lanes without a block or column read the tile's first one), so
  // that none waits in a branch before the input loads go out
  const int64_t rbs = bvalid ? rb : r0, cbs = bvalid ? cb : c0, ccs = c0 + (cvalid ? lane : 0);
  const uint32_t bsc = kFuse ? e8m0_of<T>(row_amax<T>(p, rbs, cbs))
                             : p.scale_row[rbs * p.ld_sr + (cbs >> 5)];
  uint32_t csb = 0;
  if constexpr (kCol)
    csb = kFuse ? e8m0_of<T>(static_cast<const T*>(p.amax_col)[band * p.ld_ac + ccs])
                : p.scale_col[band * p.ld_sc + ccs];
  const T* in_base = static_cast<const T*>(p.input);
  uint32_t raw[kBlockLen];
  uint32_t in = 0;
#pragma unroll
  for (int i = 0; i < kBlockLen; ++i) {
    const int64_t g0 = (r0 + i) * p.cols + c0;
    const int lo = (int)max<int64_t>(0, min<int64_t>(kElemTileCols, p.start - g0));
    const int hi = i < nrows ? (int)max<int64_t>(0, min<int64_t>(ncols, p.end - g0)) : 0;
    const bool inside = lane >= lo && lane < hi;
    const uint32_t v = load_raw(in_base, inside ? g0 - p.start + lane : 0, (int)sizeof(T));
    raw[i] = inside ? v : 0u;
    in |= (uint32_t)inside << i;
  }
  if constexpr (kFuse) {  // the scales of the blocks the fragment touches
    if (bvalid && row_block_touched(p, rb, cb)) p.scale_row[rb * p.ld_sr + (cb >> 5)] = (uint8_t)bsc;
    if constexpr (kCol) {
      if (cvalid && col_block_touched(corners_of(p), r0, r0 + nrows - 1, c0 + lane))
        p.scale_col[band * p.ld_sc + c0 + lane] = (uint8_t)csb;
    }
  }
  const int cshift = 127 - (int)csb;
#pragma unroll
  for (int i = 0; i < kBlockLen; ++i) {
    const uint32_t s0 = __builtin_amdgcn_readlane(bsc, 2 * i);
    const uint32_t s1 = __builtin_amdgcn_readlane(bsc, 2 * i + 1);
    if ((in >> i) & 1u) {
      const float w = work_value<T, kPre>(raw[i]);
      const int64_t o = (r0 + i) * p.cols + c0 - p.start;  // uniform: the row's lane 0
      p.data_row[o + lane] = cvt1(w, 127 - (int)(lane < 32 ? s0 : s1));
      if constexpr (kCol) p.data_col[o + lane] = cvt1(w, cshift);
    }
  }
}

// Single-pass quantize for any layout: a wave per (band, 64 columns), one lane per column,
// the band's 32 values of the column held in registers.
template <typename T, bool kCol, bool kPre>
__global__ __launch_bounds__(kThreads) void quantize_elem_kernel(GroupArgs ga) {
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  pin_header(ga);
  const uint32_t lt = xcd_remap(blockIdx.x, gridDim.x) * kWavesPerGroup + wave;
  const int k = piece_of(ga, lt);
  const TileArgs& p = ga.piece[k];
  pin_tile_fields(ga, k);
  const int64_t tile = (int64_t)(lt - ga.first[k]) + p.tile0;
  if (tile >= p.ntiles) return;
  const int64_t band = p.band0 + tile / p.ntc;
  const int64_t c = (tile % p.ntc) * kElemTileCols + lane;
  const int64_t r0 = band * kBlockLen;
  const bool cvalid = c < p.cols;
  const int nrows = (int)min<int64_t>(kBlockLen, p.rows - r0);
  uint32_t raw[kBlockLen];
#pragma unroll
  for (int i = 0; i < kBlockLen; ++i) {
    // every lane loads (lanes without an element read the fragment's first one), so no load
    // sits in a branch that would wait for it
    const bool valid = cvalid && i < nrows;
    const uint32_t v =
        load_raw(p.input, valid ? (r0 + i) * p.cols + c - p.start : 0, (int)sizeof(T));
    raw[i] = valid ? v : 0u;
  }
  int cshift = 0;
  if constexpr (kCol) {
    uint32_t cmax = 0;
#pragma unroll
    for (int i = 0; i < kBlockLen; ++i) cmax = umax(cmax, abs_bits<T, kPre>(raw[i]));
    const uint8_t sb = e8m0_of<T>(cmax);
    cshift = 127 - (int)sb;
    if (cvalid) {
      p.scale_col[band * p.ld_sc + c] = sb;
      if (p.amax_col) static_cast<T*>(p.amax_col)[band * p.ld_ac + c] = (T)cmax;
    }
  }
#pragma unroll
  for (int i = 0; i < kBlockLen; ++i) {
    if (i < nrows) {
      const int64_t r = r0 + i;
      const uint32_t m = half_wave_max(abs_bits<T, kPre>(raw[i]));  // the lane's row-wise block
      const uint8_t sb = e8m0_of<T>(m);
      if (cvalid && (lane & 31) == 0) {
        p.scale_row[r * p.ld_sr + (c >> 5)] = sb;
        if (p.amax_row) static_cast<T*>(p.amax_row)[r * p.ld_ar + (c >> 5)] = (T)m;
      }
      if (cvalid) {
        const float w = work_value<T, kPre>(raw[i]);
        const int64_t o = r * p.cols + c - p.start;
        p.data_row[o] = cvt1(w, 127 - (int)sb);
        if constexpr (kCol) p.data_col[o] = cvt1(w, cshift);
      }
    }
  }
}

// ------------------------------------------------------------------ E8M0 scales

struct ScaleArgs {
  int64_t rows, cols, start, end;
  const void* amax_row;
  int64_t ld_ar;
  const void* amax_col;
  int64_t ld_ac;
  uint8_t* scale_row;
  int64_t ld_sr;
  uint8_t* scale_col;
  int64_t ld_sc;
  int64_t r_first, r_last;  // rows the fragment touches
  int64_t b_first, b_last;  // bands the fragment touches
  int64_t r_lo, b_lo;       // first row / band of this launch
  uint32_t items_row;        // 8-entry items per row (row-wise part)
  uint32_t items_row_total;  // items of this launch's row-wise part
  uint32_t items_col;        // 8-entry items per band (column-wise part)
  uint32_t items_col_total;  // items of this launch's column-wise part (0 when absent)
  int32_t row_vec, col_vec;  // rows of amax / scales aligned for 16-byte / 8-byte vectors
};

// One launch covers the scale items of up to kMaxGroup pieces (or parts of pieces) of one
// dtype: workgroups first[k] .. first[k + 1] - 1 belong to part k.
struct ScaleGroup {
  ScaleArgs part[kMaxGroup];
  uint32_t first[kMaxGroup + 1];
  int32_t n;
};


// Whether column-wise block (b, c) holds an element of [start, end).
__device__ __forceinline__ bool col_block_touched(const ScaleArgs& p, int64_t b, int64_t c) {
  const int64_t r0 = b * kBlockLen;
  const int64_t r1 = min<int64_t>(r0 + kBlockLen, p.rows) - 1;
  const int64_t need = p.start - c;  // smallest row r with r * cols + c >= start
  int64_t rmin = need <= 0 ? 0 : (need + p.cols - 1) / p.cols;
  if (rmin < r0) rmin = r0;
  return rmin <= r1 && rmin * p.cols + c < p.end;
}

// One thread per 8 consecutive entries of a row (row-wise part) or of a band (column-wise
// part).  Rows and bands strictly between the fragment's first and last are wholly touched
// and, when aligned, move as one 16-byte (BF16) or two 16-byte (FP32) amax loads and one
// 8-byte scale store; the first and last row / band test each entry's block membership.
template <typename T>
__device__ __forceinline__ void scale_segment(const T* a, uint8_t* s, int64_t x0, int64_t width,
                                              bool vec) {
  if (vec && x0 + 8 <= width) {
    uint32_t w[8];
    if constexpr (sizeof(T) == 2) {
      uint32_t d[4];
      load16(a + x0, d);
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = (d[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
    } else {
      uint32_t d0[4], d1[4];
      load16(a + x0, d0);
      load16(a + x0 + 4, d1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[j] = d0[j];
        w[j + 4] = d1[j];
      }
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= (uint32_t)e8m0_of<T>(w[j]) << (8 * j);
      hi |= (uint32_t)e8m0_of<T>(w[j + 4]) << (8 * j);
    }
    *reinterpret_cast<uint2*>(s + x0) = make_uint2(lo, hi);
  } else {
    for (int64_t x = x0; x < min<int64_t>(x0 + 8, width); ++x) s[x] = e8m0_of<T>(a[x]);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void scales_kernel(ScaleGroup g) {
  int k = 0;  // the part this workgroup serves (uniform: a scalar loop)
  while (k + 1 < g.n && blockIdx.x >= g.first[k + 1]) ++k;
  const ScaleArgs& p = g.part[k];
  const uint32_t i = (blockIdx.x - g.first[k]) * 256u + threadIdx.x;
  if (i < p.items_row_total) {
    const uint32_t rr = i / p.items_row;
    const int64_t r = p.r_lo + rr;
    const int64_t x0 = (int64_t)(i - rr * p.items_row) * 8;
    const int64_t nb = (p.cols + kBlockLen - 1) / kBlockLen;
    const T* a = static_cast<const T*>(p.amax_row) + r * p.ld_ar;
    uint8_t* s = p.scale_row + r * p.ld_sr;
    if (r == p.r_first || r == p.r_last) {
      for (int64_t x = x0; x < min<int64_t>(x0 + 8, nb); ++x) {
        const int64_t gb = r * p.cols + x * kBlockLen;
        const int64_t ge = min<int64_t>(gb + kBlockLen, (r + 1) * p.cols);
        if (gb < p.end && ge > p.start) s[x] = e8m0_of<T>(a[x]);
      }
    } else {
      scale_segment<T>(a, s, x0, nb, p.row_vec);
    }
    return;
  }
  const uint32_t j = i - p.items_row_total;
  if (j >= p.items_col_total) return;
  const uint32_t bb = j / p.items_col;
  const int64_t b = p.b_lo + bb;
  const int64_t x0 = (int64_t)(j - bb * p.items_col) * 8;
  const T* a = static_cast<const T*>(p.amax_col) + b * p.ld_ac;
  uint8_t* s = p.scale_col + b * p.ld_sc;
  if (b == p.b_first || b == p.b_last) {
    for (int64_t c = x0; c < min<int64_t>(x0 + 8, p.cols); ++c)
      if (col_block_touched(p, b, c)) s[c] = e8m0_of<T>(a[c]);
  } else {
    scale_segment<T>(a, s, x0, p.cols, p.col_vec);
  }
}

// ------------------------------------------------------------------ MAX-combine

constexpr int kMaxSrcs = 8;

struct CombineArgs {
  const void* src[kMaxSrcs];
  int k;
  void* dst;
  int64_t count;   // entries
  int32_t vec;     // every pointer 16-byte aligned
};

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  constexpr int E = 16 / sizeof(T);
  int64_t done = 0;
  if (a.vec) {
    const int64_t n16 = a.count / E;
    for (int64_t i = tid; i < n16; i += stride) {
      uint32_t m[4];
      load16(static_cast<const uint4*>(a.src[0]) + i, m);
      for (int j = 1; j < a.k; ++j) {
        uint32_t v[4];
        load16(static_cast<const uint4*>(a.src[j]) + i, v);
#pragma unroll
        for (int t = 0; t < 4; ++t) m[t] = sizeof(T) == 2 ? pk_max_u16(m[t], v[t]) : umax(m[t], v[t]);
      }
      static_cast<uint4*>(a.dst)[i] = make_uint4(m[0], m[1], m[2], m[3]);
    }
    done = n16 * E;
  }
  for (int64_t i = done + tid; i < a.count; i += stride) {
    uint32_t m = static_cast<const T*>(a.src[0])[i];
    for (int j = 1; j < a.k; ++j) m = umax(m, static_cast<const T*>(a.src[j])[i]);
    static_cast<T*>(a.dst)[i] = (T)m;
  }
}

// ------------------------------------------------------------------ launch helpers

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

TileArgs tile_args(const Piece& p, int64_t tile_cols) {
  TileArgs a{};
  a.rows = p.rows;
  a.cols = p.cols;
  a.start = p.start;
  a.end = p.start + p.len;
  a.input = p.input;
  a.amax_row = p.amax_row;
  a.ld_ar = p.ld_ar;
  a.amax_col = p.amax_col;
  a.ld_ac = p.ld_ac;
  a.scale_row = p.scale_row;
  a.ld_sr = p.ld_sr;
  a.scale_col = p.scale_col;
  a.ld_sc = p.ld_sc;
  a.data_row = p.data_row;
  a.data_col = p.data_col;
  const int64_t b0 = (p.start / p.cols) / kBlockLen;
  const int64_t b1 = ((a.end - 1) / p.cols) / kBlockLen;
  a.band0 = b0;
  a.ntc = cdiv(p.cols, tile_cols);
  a.ntiles = (b1 - b0 + 1) * a.ntc;
  const int64_t esz = elem_size(p.dtype);
  a.col_vec = p.amax_col && (reinterpret_cast<uintptr_t>(p.amax_col) % 16 == 0) &&
              ((p.ld_ac * esz) % 16 == 0);
  a.row_vec = p.amax_row && (reinterpret_cast<uintptr_t>(p.amax_row) % 16 == 0) &&
              ((p.ld_ar * esz) % 16 == 0);
  a.row_pair = p.amax_row && (reinterpret_cast<uintptr_t>(p.amax_row) % 4 == 0) &&
               ((p.ld_ar * esz) % 4 == 0);
  a.col_pair = p.amax_col && (reinterpret_cast<uintptr_t>(p.amax_col) % 4 == 0) &&
               ((p.ld_ac * esz) % 4 == 0);
  const uintptr_t virt = reinterpret_cast<uintptr_t>(p.input) - (uintptr_t)(p.start * esz);
  a.in_shift2 = (virt % 4) == 2;
  auto mis = [&](const uint8_t* d) {
    return d ? (int32_t)((reinterpret_cast<uintptr_t>(d) - (uintptr_t)p.start) % 4) : 0;
  };
  a.mo_row = mis(p.data_row);
  a.mo_col = mis(p.data_col);
  auto lines = [&](const uint8_t* d) {
    return (int32_t)(d && (reinterpret_cast<uintptr_t>(d) - (uintptr_t)p.start) % 64 == 0 &&
                     p.cols % 64 == 0);
  };
  a.nt_row = lines(p.data_row);
  a.nt_col = lines(p.data_col);
  const int64_t e = 16 / esz;  // elements per 16-byte chunk
  a.sc_vec = p.scale_col && (reinterpret_cast<uintptr_t>(p.scale_col) % e == 0) && (p.ld_sc % e == 0);
  return a;
}

inline int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Tile arguments of the line-owned cast tiles (see cast_lines_kernel): virtual rows
// v = floor((g - shift) / cols) from the fragment's first to its last element, in bands of 32.
TileArgs tile_args_lines(const Piece& p, int64_t tile_cols, int64_t shift) {
  TileArgs a = tile_args(p, tile_cols);
  const int64_t end = p.start + p.len;
  const int64_t b0 = floor_div(floor_div(p.start - shift, p.cols), kBlockLen);
  const int64_t b1 = floor_div(floor_div(end - 1 - shift, p.cols), kBlockLen);
  a.shift = (int32_t)shift;
  a.band0 = b0;
  a.ntiles = (b1 - b0 + 1) * a.ntc;
  const int64_t esz = elem_size(p.dtype);
  const uintptr_t virt = reinterpret_cast<uintptr_t>(p.input) - (uintptr_t)(p.start * esz);
  a.in_shift2 = ((virt + (uintptr_t)(shift * esz)) % 4) == 2;
  return a;
}

// LDS bytes per CU of the current device (160 KiB on MI355X), queried once per device; 0 if
// unknown.
int lds_per_cu() {
  static std::atomic<int> cache[64];  // 0: not queried yet; -1: unknown
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
        hipSuccess) {
      (void)hipGetLastError();  // a failed query only drops the cap; the launch check stays clean
      v = -1;
    }
    if (v <= 0) v = -1;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}

// Dynamic LDS bytes that hold `kernel` at `cap` resident workgroups per CU (0: no cap).
template <typename K>
size_t cap_lds(K kernel, int cap) {
  const int lds = lds_per_cu();
  if (cap <= 0 || lds <= 0) return 0;
  static std::mutex mu;  // static LDS of each kernel, from its attributes, looked up once
  static std::unordered_map<const void*, size_t> static_lds;
  const void* key = reinterpret_cast<const void*>(kernel);
  size_t st;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = static_lds.find(key);
    if (it == static_lds.end()) {
      hipFuncAttributes a{};
      if (hipFuncGetAttributes(&a, key) == hipSuccess) {
        st = a.sharedSizeBytes;
      } else {
        (void)hipGetLastError();  // as above
        st = 0;
      }
      static_lds.emplace(key, st);
    } else {
      st = it->second;
    }
  }
  const size_t per = (size_t)lds / (size_t)cap;
  return per > st ? per - st : 0;
}

// Launches `kernel` over the tiles of `ps`, kMaxGroup pieces per launch.  tiles_per_wg is 1
// for the vector kernels (a workgroup per tile) and kWavesPerGroup for the element-wise ones
// (a wave per tile).  Launches under kSmallLaunchTiles tiles run `small_kernel`; the others
// run `kernel`, held at `cap` resident workgroups per CU (0: no cap).
// One kernel launch.  With a call being timed (mxfp8_time_next_call) the launch goes through
// hipExtLaunchKernel, whose events the runtime stamps when the kernel itself starts and ends:
// the call's first kernel records the start event, every kernel the stop event.
template <typename F, typename... A>
hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, size_t shm, hipStream_t s, A... args) {
  CallEvents& ev = call_events();
  if (ev.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shm, s, ev.start, ev.stop, 0, args...);
    ev.start = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
  }
  return hipGetLastError();
}

// A kernel for launches of fewer than `below` tiles: it takes each tile as `split` workgroups
// of `threads` threads (the cast's split tiles, the amax's wide workgroups).  `one` is the same
// kernel for a launch of a single piece (kOne): its piece index is known, so the workgroup
// loads the launch header and the piece's fields in one batch of scalar loads, one round trip
// where the piece lookup takes two (graph replays, 1024x1024 calls: 3-7% faster).
template <typename K>
struct Tier {
  K kernel = nullptr;
  int64_t below = 0;
  int split = 1;
  int threads = kThreads;
  K one = nullptr;
};

template <typename K>
hipError_t launch_grouped(K kernel, K small_kernel, const std::vector<TileArgs>& ps,
                          int tiles_per_wg, int cap, hipStream_t s, Tier<K> t1 = {},
                          Tier<K> t2 = {}) {
  for (size_t i0 = 0; i0 < ps.size(); i0 += kMaxGroup) {
    GroupArgs g{};
    g.n = (int32_t)std::min<size_t>(kMaxGroup, ps.size() - i0);
    int64_t first[kMaxGroup], total = 0;
    for (int k = 0; k < g.n; ++k) total += ps[i0 + k].ntiles;
    // A launch of few tiles leaves most of the GPU idle: the first tier (t1, then t2) whose
    // bound it stays under runs it, with the pieces' tile counts scaled by its split.
    const Tier<K> tier = t1.kernel != nullptr && total < t1.below   ? t1
                         : t2.kernel != nullptr && total < t2.below ? t2
                                                                    : Tier<K>{};
    const int split = tier.split;
    total = 0;
    for (int k = 0; k < g.n; ++k) {
      g.piece[k] = ps[i0 + k];
      g.piece[k].ntiles *= split;
      if (g.piece[k].ntiles > 0xFFFFFFFFll) return hipErrorInvalidConfiguration;  // 32-bit tile ids
      first[k] = total;
      // element-wise tiles start on a workgroup boundary so each workgroup has one piece
      total += cdiv(g.piece[k].ntiles, tiles_per_wg) * tiles_per_wg;
    }
    const int64_t groups = cdiv(total, tiles_per_wg);
    const bool small = total < kSmallLaunchTiles;
    const K tk = g.n == 1 && tier.one != nullptr ? tier.one : tier.kernel;
    const K k = tk != nullptr ? tk : small ? small_kernel : kernel;
    const size_t shm = small ? 0 : cap_lds(k, cap);
    for (int64_t g0 = 0; g0 < groups; g0 += kMaxLaunchGroups) {
      // the pieces' first tiles counted from this launch's first workgroup (see GroupArgs)
      const int64_t base = g0 * tiles_per_wg;
      for (int j = g.n; j < kMaxGroup; ++j) g.first[j] = kNoPiece;
      for (int j = 0; j < g.n; ++j) {
        const int64_t f = first[j] - base;
        g.first[j] = f <= 0 ? 0u : (f >= (int64_t)kNoPiece ? kNoPiece : (uint32_t)f);
        g.piece[j].tile0 = f < 0 ? -f : 0;
      }
      const int64_t ng = std::min<int64_t>(kMaxLaunchGroups, groups - g0);
      const hipError_t e = launch_kernel(k, dim3((unsigned)ng), dim3(tier.threads), shm, s, g);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}


// Pieces of one call, bucketed by kernel specialization: dtype x column-wise x pre-round x
// vector path.
struct Buckets {
  std::vector<TileArgs> b[2][2][2][2];  // [bf16][col][pre][vec]
};

// The vector-path pieces of both directions, for one kernel with run-time guards.
inline std::vector<TileArgs> both_directions(const Buckets& bk, int bf16, int pre) {
  std::vector<TileArgs> v = bk.b[bf16][1][pre][1];
  v.insert(v.end(), bk.b[bf16][0][pre][1].begin(), bk.b[bf16][0][pre][1].end());
  return v;
}

// Whether a call's vector pieces of one element type hold both directions in fewer than
// kSmallLaunchTiles tiles.  Such a call (one rank's share of a batch of row-only and
// bidirectional weights) goes out as one launch of the kernel that selects the column-wise
// work per piece at run time: one launch's fixed cost is most of a small call's time, and the
// run-time selection costs little next to it (one rank's layer-batch fragment: amax 16.6 ->
// 14.2 us, cast 21.8 -> 19.9 us).  Larger calls keep one compile-time specialized launch per
// direction, which there measured faster (layer-batch cast 119.5 against 126.5 us).
inline bool one_launch_for_both(const Buckets& bk, int bf16, int pre) {
  const std::vector<TileArgs>& c = bk.b[bf16][1][pre][1];
  const std::vector<TileArgs>& r = bk.b[bf16][0][pre][1];
  if (c.empty() || r.empty()) return false;
  int64_t tiles = 0;
  for (const TileArgs& t : c) tiles += t.ntiles;
  for (const TileArgs& t : r) tiles += t.ntiles;
  return tiles < kSmallLaunchTiles;
}

// The pieces of one amax launch (or of launches that may run in any order), each with its
// amax_own flag: set where no other of them has the same row-wise or column-wise amax array
// (pieces of one call share amax arrays only as the same pointer in the same role).
inline std::vector<TileArgs> mark_amax_owners(std::vector<TileArgs> v) {
  std::unordered_map<const void*, int> uses;
  for (const TileArgs& t : v) {
    if (t.amax_row) ++uses[t.amax_row];
    if (t.amax_col) ++uses[t.amax_col];
  }
  for (TileArgs& t : v)
    t.amax_own = (!t.amax_row || uses[t.amax_row] == 1) && (!t.amax_col || uses[t.amax_col] == 1);
  return v;
}

template <typename T, bool kCol, bool kPre>
hipError_t launch_amax_bucket(const std::vector<TileArgs>& vec, const std::vector<TileArgs>& elem,
                              hipStream_t s) {
  hipError_t e = hipSuccess;
  if (!vec.empty())
    e = launch_grouped(amax_vec_kernel<T, kCol, kPre, Occupancy<T>::kAmax>,
                       amax_vec_kernel<T, kCol, kPre, Occupancy<T>::kAmaxSmall>,
                       mark_amax_owners(vec), 1,
                       Occupancy<T>::kAmaxCap, s,
                       {amax_vec_kernel<T, kCol, kPre, Occupancy<T>::kAmaxSmall, false, 8>,
                        kAmax8Tiles, 1, kWaveSize * 8,
                        amax_vec_kernel<T, kCol, kPre, Occupancy<T>::kAmaxSmall, false, 8, true>},
                       {amax_vec_kernel<T, kCol, kPre, Occupancy<T>::kAmaxSmall>, kSmallLaunchTiles,
                        1, kThreads,
                        amax_vec_kernel<T, kCol, kPre, Occupancy<T>::kAmaxSmall, false,
                                        kWavesPerGroup, true>});
  if (e == hipSuccess && !elem.empty())
    e = launch_grouped(amax_elem_kernel<T, kCol, kPre>, amax_elem_kernel<T, kCol, kPre>, elem,
                       kWavesPerGroup, 0, s);
  return e;
}

template <typename T, bool kCol, bool kPre, bool kFuse>
hipError_t launch_cast_bucket(const std::vector<TileArgs>& vec, const std::vector<TileArgs>& elem,
                              hipStream_t s) {
  hipError_t e = hipSuccess;
  // large bidirectional BF16 launches load the scale bytes first (cast_vec_kernel's
  // kScaleFirst; the row-only cast measured 0.8% slower with it)
  constexpr bool kSF = sizeof(T) == 2 && kCol && !kFuse;
  // launches too small to fill the GPU cast split tiles (cast_vec_kernel's kSplit)
  if (!vec.empty())
    e = launch_grouped(cast_vec_kernel<T, kCol, kPre, kFuse, Occupancy<T>::kCast, false, kSF>,
                       cast_vec_kernel<T, kCol, kPre, kFuse, Occupancy<T>::kCast>, vec, 1,
                       Occupancy<T>::cast_cap(kCol, kFuse), s,
                       {cast_vec_kernel<T, kCol, kPre, kFuse, Occupancy<T>::kCast, false, false, 8>,
                        kSplit8Tiles, 8, kThreads,
                        cast_vec_kernel<T, kCol, kPre, kFuse, Occupancy<T>::kCast, false, false, 8,
                                        true>},
                       {cast_vec_kernel<T, kCol, kPre, kFuse, Occupancy<T>::kCast, false, false, 4>,
                        kSplit4Tiles, 4, kThreads,
                        cast_vec_kernel<T, kCol, kPre, kFuse, Occupancy<T>::kCast, false, false, 4,
                                        true>});
  if (e == hipSuccess && !elem.empty())
    e = launch_grouped(cast_elem_kernel<T, kCol, kPre, kFuse>, cast_elem_kernel<T, kCol, kPre, kFuse>,
                       elem, kWavesPerGroup, 0, s);
  return e;
}

template <typename T, bool kCol, bool kPre>
hipError_t launch_lines_bucket(const std::vector<TileArgs>& ps, hipStream_t s) {
  if (ps.empty()) return hipSuccess;
  return launch_grouped(cast_lines_kernel<T, kCol, kPre, Occupancy<T>::kCast>,
                        cast_lines_kernel<T, kCol, kPre, Occupancy<T>::kCast>, ps, 1,
                        Occupancy<T>::cast_cap(kCol, false), s);
}

template <typename T, bool kPre>
hipError_t launch_cast_guarded(const Buckets& bk, hipStream_t s) {
  const int bf16 = sizeof(T) == 2, pre = kPre;
  const std::vector<TileArgs> v = both_directions(bk, bf16, pre);
  hipError_t e = hipSuccess;
  if (!v.empty())
    e = launch_grouped(  // one kernel for both directions: it takes the bidirectional order
        cast_vec_kernel<T, true, kPre, false, Occupancy<T>::kCast, true, sizeof(T) == 2>,
        cast_vec_kernel<T, true, kPre, false, Occupancy<T>::kCast, true>, v, 1,
        Occupancy<T>::cast_cap(true, false), s,
        {cast_vec_kernel<T, true, kPre, false, Occupancy<T>::kCast, true, false, 8>, kSplit8Tiles, 8,
         kThreads, cast_vec_kernel<T, true, kPre, false, Occupancy<T>::kCast, true, false, 8, true>},
        {cast_vec_kernel<T, true, kPre, false, Occupancy<T>::kCast, true, false, 4>, kSplit4Tiles, 4,
         kThreads, cast_vec_kernel<T, true, kPre, false, Occupancy<T>::kCast, true, false, 4, true>});
  const std::vector<TileArgs> none;
  if (e == hipSuccess) e = launch_cast_bucket<T, true, kPre, false>(none, bk.b[bf16][1][pre][0], s);
  if (e == hipSuccess) e = launch_cast_bucket<T, false, kPre, false>(none, bk.b[bf16][0][pre][0], s);
  return e;
}

// The casts of one element type and pre-round setting: with run-time guards (the ablation
// library, or a small call holding both directions) one kernel for the vector pieces of both
// directions, else one compile-time specialized launch per direction.
template <typename T, bool kPre, bool kFuse>
hipError_t launch_cast_dtype(const Buckets& bk, hipStream_t s) {
  const int bf16 = sizeof(T) == 2, pre = kPre;
  if constexpr (!kFuse) {
    if (kRuntimeGuards || one_launch_for_both(bk, bf16, pre))
      return launch_cast_guarded<T, kPre>(bk, s);
  }
  hipError_t e = launch_cast_bucket<T, true, kPre, kFuse>(bk.b[bf16][1][pre][1], bk.b[bf16][1][pre][0], s);
  if (e == hipSuccess)
    e = launch_cast_bucket<T, false, kPre, kFuse>(bk.b[bf16][0][pre][1], bk.b[bf16][0][pre][0], s);
  return e;
}

template <bool kFuse>
hipError_t launch_cast_pieces(const Piece* ps, int n, hipStream_t s) {
  Buckets bk, lines;  // lines: pieces of the plain cast that take the line-owned tiles
  for (int i = 0; i < n; ++i) {
    const Piece& p = ps[i];
    const bool vec = vec_common_ok(p);
    const int64_t width = vec ? kWaveSize * (16 / elem_size(p.dtype)) : kElemTileCols;
    const int64_t shift = kFuse ? 0 : line_shift(p);
    if (shift)
      lines.b[p.dtype == kBF16][p.data_col != nullptr][p.preround][1].push_back(
          tile_args_lines(p, width, shift));
    else
      bk.b[p.dtype == kBF16][p.data_col != nullptr][p.preround][vec].push_back(tile_args(p, width));
  }
  hipError_t e = hipSuccess;  // each launch only if everything before it went out
  if (e == hipSuccess) e = launch_cast_dtype<uint16_t, false, kFuse>(bk, s);
  if (e == hipSuccess) e = launch_cast_dtype<uint32_t, false, kFuse>(bk, s);
  if (e == hipSuccess) e = launch_cast_dtype<uint32_t, true, kFuse>(bk, s);
  if constexpr (!kFuse) {
    if (e == hipSuccess) e = launch_lines_bucket<uint16_t, true, false>(lines.b[1][1][0][1], s);
    if (e == hipSuccess) e = launch_lines_bucket<uint16_t, false, false>(lines.b[1][0][0][1], s);
    if (e == hipSuccess) e = launch_lines_bucket<uint32_t, true, false>(lines.b[0][1][0][1], s);
    if (e == hipSuccess) e = launch_lines_bucket<uint32_t, false, false>(lines.b[0][0][0][1], s);
    if (e == hipSuccess) e = launch_lines_bucket<uint32_t, true, true>(lines.b[0][1][1][1], s);
    if (e == hipSuccess) e = launch_lines_bucket<uint32_t, false, true>(lines.b[0][0][1][1], s);
  }
  return e;
}

}  // namespace

template <typename T, bool kPre>
hipError_t launch_amax_guarded(const Buckets& bk, hipStream_t s) {
  const int bf16 = sizeof(T) == 2, pre = kPre;
  const std::vector<TileArgs> v = mark_amax_owners(both_directions(bk, bf16, pre));
  hipError_t e = hipSuccess;
  if (!v.empty())
    e = launch_grouped(amax_vec_kernel<T, true, kPre, Occupancy<T>::kAmax, true>,
                       amax_vec_kernel<T, true, kPre, Occupancy<T>::kAmaxSmall, true>, v, 1,
                       Occupancy<T>::kAmaxCap, s,
                       {amax_vec_kernel<T, true, kPre, Occupancy<T>::kAmaxSmall, true, 8>,
                        kAmax8Tiles, 1, kWaveSize * 8,
                        amax_vec_kernel<T, true, kPre, Occupancy<T>::kAmaxSmall, true, 8, true>},
                       {amax_vec_kernel<T, true, kPre, Occupancy<T>::kAmaxSmall, true>,
                        kSmallLaunchTiles, 1, kThreads,
                        amax_vec_kernel<T, true, kPre, Occupancy<T>::kAmaxSmall, true,
                                        kWavesPerGroup, true>});
  // the element-wise kernels keep their compile-time specializations
  const std::vector<TileArgs> none;
  if (e == hipSuccess) e = launch_amax_bucket<T, true, kPre>(none, bk.b[bf16][1][pre][0], s);
  if (e == hipSuccess) e = launch_amax_bucket<T, false, kPre>(none, bk.b[bf16][0][pre][0], s);
  return e;
}

// The amax of one element type and pre-round setting, dispatched as the cast's
// (launch_cast_dtype).
template <typename T, bool kPre>
hipError_t launch_amax_dtype(const Buckets& bk, hipStream_t s) {
  const int bf16 = sizeof(T) == 2, pre = kPre;
  if (kRuntimeGuards || one_launch_for_both(bk, bf16, pre)) return launch_amax_guarded<T, kPre>(bk, s);
  hipError_t e = launch_amax_bucket<T, true, kPre>(bk.b[bf16][1][pre][1], bk.b[bf16][1][pre][0], s);
  if (e == hipSuccess) e = launch_amax_bucket<T, false, kPre>(bk.b[bf16][0][pre][1], bk.b[bf16][0][pre][0], s);
  return e;
}

hipError_t launch_amax_buckets(const Buckets& bk, hipStream_t s) {
  hipError_t e = hipSuccess;  // each launch only if everything before it went out
  if (e == hipSuccess) e = launch_amax_dtype<uint16_t, false>(bk, s);
  if (e == hipSuccess) e = launch_amax_dtype<uint32_t, false>(bk, s);
  if (e == hipSuccess) e = launch_amax_dtype<uint32_t, true>(bk, s);
  return e;
}

hipError_t launch_partial_amax(const Piece* ps, int n, hipStream_t s) {
  Buckets bk;
  for (int i = 0; i < n; ++i) {
    const Piece& p = ps[i];
    const bool vec = amax_fast_ok(p);
    const int64_t width = vec ? kWaveSize * (16 / elem_size(p.dtype)) : kElemTileCols;
    bk.b[p.dtype == kBF16][p.amax_col != nullptr][p.preround][vec].push_back(tile_args(p, width));
  }
  return launch_amax_buckets(bk, s);
}

template <typename T, bool kCol, bool kPre>
hipError_t launch_quantize_bucket(const std::vector<TileArgs>& vec,
                                  const std::vector<TileArgs>& elem, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (!vec.empty())
    e = launch_grouped(quantize_vec_kernel<T, kCol, kPre, Occupancy<T>::kCast>,
                       quantize_vec_kernel<T, kCol, kPre, Occupancy<T>::kCast>, vec, 1,
                       Occupancy<T>::kQuantCap, s,
                       // launches too small to fill the GPU: 8-wave workgroups, as the amax's
                       {quantize_vec_kernel<T, kCol, kPre, Occupancy<T>::kAmaxSmall, 8>,
                        kAmax8Tiles, 1, kWaveSize * 8,
                        quantize_vec_kernel<T, kCol, kPre, Occupancy<T>::kAmaxSmall, 8, true>});
  if (e == hipSuccess && !elem.empty())
    e = launch_grouped(quantize_elem_kernel<T, kCol, kPre>, quantize_elem_kernel<T, kCol, kPre>,
                       elem, kWavesPerGroup, 0, s);
  return e;
}

hipError_t launch_quantize(const Piece* ps, int n, hipStream_t s) {
  Buckets bk;
  for (int i = 0; i < n; ++i) {
    const Piece& p = ps[i];
    const bool vec = vec_common_ok(p);
    const int64_t width = vec ? kWaveSize * (16 / elem_size(p.dtype)) : kElemTileCols;
    bk.b[p.dtype == kBF16][p.data_col != nullptr][p.preround][vec].push_back(tile_args(p, width));
  }
  hipError_t e = hipSuccess;  // each launch only if everything before it went out
  if (e == hipSuccess) e = launch_quantize_bucket<uint16_t, true, false>(bk.b[1][1][0][1], bk.b[1][1][0][0], s);
  if (e == hipSuccess) e = launch_quantize_bucket<uint16_t, false, false>(bk.b[1][0][0][1], bk.b[1][0][0][0], s);
  if (e == hipSuccess) e = launch_quantize_bucket<uint32_t, true, false>(bk.b[0][1][0][1], bk.b[0][1][0][0], s);
  if (e == hipSuccess) e = launch_quantize_bucket<uint32_t, false, false>(bk.b[0][0][0][1], bk.b[0][0][0][0], s);
  if (e == hipSuccess) e = launch_quantize_bucket<uint32_t, true, true>(bk.b[0][1][1][1], bk.b[0][1][1][0], s);
  if (e == hipSuccess) e = launch_quantize_bucket<uint32_t, false, true>(bk.b[0][0][1][1], bk.b[0][0][1][0], s);
  return e;
}

hipError_t launch_partial_cast(const Piece* ps, int n, hipStream_t s) {
  return launch_cast_pieces<false>(ps, n, s);
}

hipError_t launch_scales_and_cast(const Piece* ps, int n, hipStream_t s) {
  return launch_cast_pieces<true>(ps, n, s);
}

// Items (threads) per part of a scales launch beyond which a fragment's scales are split into
// parts of whole rows, then whole bands, well below the 2^32 work-items a dispatch holds.
constexpr int64_t kMaxScaleItems = int64_t(1) << 24;

// The scale parts of one piece: usually one; larger fragments are split into parts of whole
// rows and of whole bands, each within kMaxScaleItems.
hipError_t scale_parts(const Piece& p, std::vector<ScaleArgs>& out) {
  ScaleArgs a{};
  a.rows = p.rows;
  a.cols = p.cols;
  a.start = p.start;
  a.end = p.start + p.len;
  a.amax_row = p.amax_row;
  a.ld_ar = p.ld_ar;
  a.amax_col = p.amax_col;
  a.ld_ac = p.ld_ac;
  a.scale_row = p.scale_row;
  a.ld_sr = p.ld_sr;
  a.scale_col = p.scale_col;
  a.ld_sc = p.ld_sc;
  a.r_first = p.start / p.cols;
  a.r_last = (a.end - 1) / p.cols;
  a.b_first = a.r_first / kBlockLen;
  a.b_last = a.r_last / kBlockLen;
  const bool col = p.amax_col != nullptr;
  const int64_t esz = elem_size(p.dtype);
  const int64_t nb = cdiv(p.cols, kBlockLen);
  const int64_t items_row = cdiv(nb, 8), items_col = cdiv(p.cols, 8);
  const int64_t nrows = a.r_last - a.r_first + 1, nbands = a.b_last - a.b_first + 1;
  // a part holds at least one whole row or band: at most 2^31 items
  constexpr int64_t kMaxRowItems = int64_t(1) << 31;
  if (items_row > kMaxRowItems || (col && items_col > kMaxRowItems))
    return hipErrorInvalidConfiguration;
  a.items_row = (uint32_t)items_row;
  a.items_col = (uint32_t)items_col;
  auto aligned = [](const void* q, int64_t n) { return reinterpret_cast<uintptr_t>(q) % n == 0; };
  a.row_vec = aligned(p.amax_row, 16) && (p.ld_ar * esz) % 16 == 0 && aligned(p.scale_row, 8) &&
              p.ld_sr % 8 == 0;
  a.col_vec = col && aligned(p.amax_col, 16) && (p.ld_ac * esz) % 16 == 0 &&
              aligned(p.scale_col, 8) && p.ld_sc % 8 == 0;
  auto part = [&](int64_t r_lo, int64_t nr, int64_t b_lo, int64_t nbd) {
    a.r_lo = r_lo;
    a.b_lo = b_lo;
    a.items_row_total = (uint32_t)(nr * items_row);
    a.items_col_total = (uint32_t)(nbd * items_col);
    out.push_back(a);
  };
  const int64_t ncol = col ? nbands : 0;
  if (nrows * items_row + ncol * items_col <= kMaxScaleItems) {  // the usual case: one part
    part(a.r_first, nrows, a.b_first, ncol);
    return hipSuccess;
  }
  const int64_t rows_per = std::max<int64_t>(1, kMaxScaleItems / items_row);
  for (int64_t r = a.r_first; r <= a.r_last; r += rows_per)
    part(r, std::min(rows_per, a.r_last - r + 1), 0, 0);
  const int64_t bands_per = std::max<int64_t>(1, kMaxScaleItems / items_col);
  for (int64_t b = a.b_first; col && b <= a.b_last; b += bands_per)
    part(0, 0, b, std::min(bands_per, a.b_last - b + 1));
  return hipSuccess;
}

// The scales of every piece of a call: one launch per dtype for up to kMaxGroup parts.
hipError_t launch_compute_scales(const Piece* ps, int n, hipStream_t s) {
  std::vector<ScaleArgs> parts[2];  // [bf16]
  for (int i = 0; i < n; ++i) {
    const hipError_t e = scale_parts(ps[i], parts[ps[i].dtype == kBF16]);
    if (e != hipSuccess) return e;
  }
  // a launch stays within 2^23 workgroups (2^31 work-items); one part alone is at most 2^31
  // items (a single row or band of the widest weights), so it always fits
  constexpr int64_t kMaxScaleLaunchGroups = int64_t(1) << 23;
  for (int bf16 = 1; bf16 >= 0; --bf16) {
    const std::vector<ScaleArgs>& v = parts[bf16];
    for (size_t i0 = 0; i0 < v.size();) {
      ScaleGroup g{};
      int64_t wg = 0;
      while (g.n < kMaxGroup && i0 < v.size()) {
        const int64_t w = cdiv((int64_t)v[i0].items_row_total + v[i0].items_col_total, 256);
        if (g.n > 0 && wg + w > kMaxScaleLaunchGroups) break;
        g.part[g.n] = v[i0++];
        g.first[g.n++] = (uint32_t)wg;
        wg += w;
      }
      g.first[g.n] = (uint32_t)wg;
      if (wg == 0) continue;
      const hipError_t e =
          bf16 ? launch_kernel(scales_kernel<uint16_t>, dim3(wg), dim3(256), 0, s, g)
               : launch_kernel(scales_kernel<uint32_t>, dim3(wg), dim3(256), 0, s, g);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_combine(void* dst, const void* const* srcs, int k, int64_t count, int dtype,
                          hipStream_t s) {
  const int64_t esz = elem_size(dtype);
  // More than kMaxSrcs sources: fold them into dst kMaxSrcs - 1 at a time after the first pass.
  int done = 0;
  while (done < k) {
    CombineArgs a{};
    int n = 0;
    if (done > 0) a.src[n++] = dst;
    while (n < kMaxSrcs && done < k) a.src[n++] = srcs[done++];
    a.k = n;
    a.dst = dst;
    a.count = count;
    bool vec = reinterpret_cast<uintptr_t>(dst) % 16 == 0;
    for (int j = 0; j < n; ++j) vec = vec && reinterpret_cast<uintptr_t>(a.src[j]) % 16 == 0;
    a.vec = vec;
    const int64_t work = vec ? cdiv(count * esz, 16) : count;
    const int64_t groups = std::max<int64_t>(1, std::min<int64_t>(cdiv(work, 256), 256 * 16));
    const hipError_t e =
        dtype == kBF16
            ? launch_kernel(combine_kernel<uint16_t>, dim3((unsigned)groups), dim3(256), 0, s, a)
            : launch_kernel(combine_kernel<uint32_t>, dim3((unsigned)groups), dim3(256), 0, s, a);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mxfp8
