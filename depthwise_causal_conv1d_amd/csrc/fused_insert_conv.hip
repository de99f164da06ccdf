// fused_insert_conv.hip -- single-launch insert + depthwise causal conv over
// a paged cache (one conv stream, or all streams of a layer), for gfx950.
//
// Source: vLLM page "vllm.models.inkling.nvidia.ops.sconv", module
// description and function fused_sconv.  Per row: the input row is copied
// to the row's cache slot, and the W taps ending at the row's absolute
// position are convolved; taps inside the current forward come from the
// immutable input x, earlier taps from the paged cache via the block table.
// The slot written in a call is never read in that call, so one launch
// serves prefill, decode and speculative rows alike.
//
// Work decomposition (MI355X):
//   * one wave64 owns a tile of BT consecutive rows x a slab of 64*VEC
//     channels; each lane owns VEC consecutive channels (16 bytes: 8 bf16 or
//     4 fp32), so every x / out row access of a wave is one contiguous
//     coalesced segment and every cache access is 16 bytes per lane;
//   * the values a wave needs before its first load (metadata pointers,
//     row count, request divider, slab count, ...) arrive as leading scalar
//     kernel arguments that the hardware preloads into SGPRs;
//   * the row index is wave-uniform: a tile's positions, slots and request
//     data arrive in one per-lane gather and are broadcast to SGPRs, block-
//     table entries come through scalar registers, and every PAD / same-
//     forward / pre-forward decision is a uniform branch;
//   * the W-1 previous input rows a tap needs stay in the lane's registers:
//     rows inside the tile are the tile's own loads, rows before the tile
//     (the halo, at most W-1) come from the previous wave of the workgroup
//     through LDS, or are loaded once per tile only when a row of the tile
//     reads them;
//   * decode-shaped launches (requests of a few rows each) guess each row's
//     request and check the guess against two offsets, and with one row per
//     request read the row's block-table row ahead; their history rows,
//     pieces of 128-byte lines, are loaded as streaming reads;
//   * fp32 FMA accumulation in VGPRs, SiLU via exp2 + reciprocal, bf16
//     rounding by v_cvt_pk_bf16_f32 (round to nearest even);
//   * the grid depends only on T and C, so the decode path replays under a
//     hipGraph without any data-dependent shape.
#include "gather_window.h"
#include "sconv_device.h"
#include "sconv_host.h"

#include <type_traits>

namespace sconv {

// One conv stream of a layer: its own input, weights and output, and the
// sub-range [off_s, off_s + ws) of every head's D columns in the shared
// cache.  Its slabs are global slabs [slab0, slab0 + ceil(C / lane width)).
constexpr int kMaxStreams = 4;
struct FusedStream {
  const void* x;
  const void* w;
  void* out;
  int64_t x_rs, out_rs, w_sc, w_sk;
  int32_t C, ws, off_s, slab0;
  int32_t silu, residual;
};

struct FusedParams {
  // The kernel takes the launch geometry, the metadata and block-table
  // pointers and the request divider from its leading arguments (built
  // from these fields by launch_fused); the rest it reads here.
  uint32_t num_groups;      // grid size in workgroups
  int32_t waves_per_group;  // workgroup size / 64
  int32_t num_slabs;        // over all streams
  int32_t num_streams;
  int32_t N;
  // Division by N of non-negative 32-bit positions and slots, branch-free:
  // q = (t + ((v - t) >> n_s1)) >> n_s2 with t = mulhi(v, n_magic)
  // (Granlund & Montgomery, round-up variant; exact for every uint32 v).
  // N = 1: (0, 0, 0); N = 2^k: (1, 1, k-1); otherwise the magic number.
  uint32_t n_magic, n_s1, n_s2;
  int32_t num_reqs;         // with qsl
  int32_t nt_x;             // host choice: streaming input loads (one wave generation)
  int32_t guess;            // host choice: kQslGuess (row t's request guessed as t / k)
  uint32_t k_magic, k_s1, k_s2;  // division by k = rows per request (same scheme as N)
  int32_t bt_pref;          // block-table entries of row t read ahead (kQslGuess; 0: off)
  int32_t nt_hist;          // host choice: streaming history loads (one-row tiles)
  int32_t early_insert;     // host choice: cache inserts issued behind the history loads
  void* cache;
  const int64_t* positions;
  const int32_t* bt;
  const int32_t* seq_idx;   // per-row request (NULL: search qsl)
  const int64_t* slot;
  const int32_t* qs;        // per-row request start (NULL: search qsl)
  const int32_t* qsl;       // request row offsets [num_reqs + 1] (or NULL)
  int64_t cs0, cs1, cs2, bt_rs, T;
  int64_t num_tiles;
#if SCONV_FUSED_STRIDE
  int32_t walk_per_slab;    // striding launches: waves per slab
#endif
  FusedStream st[kMaxStreams];
};

// A fused launch that also runs a conditional window gather: workgroups
// [0, num_groups) are the conv's, the next g_groups the gather's, one per
// (slot, channel block) item in slot-major order.  The conv's come first:
// its one generation of waves starts its latency chains at once, and the
// gather's workgroups take the room its resident waves leave, then its
// tail.  (Measured on the 512 x 4-draft step: 16.0 us per launch; gather
// workgroups first 18.2 us; a few gather workgroups looping over the items
// beside the conv 17.0 us; two launches 18.3 us; gather workgroups spread
// among the conv's, SCONV_FUSED_GATHER_INTERLEAVE, 21.0 against 16.3 us.)
struct FusedGatherParams : FusedParams {
  GatherParams g;
  int32_t g_dc;      // window length d_conv, 1..4
  uint32_t g_groups;
  // Interleaved order (SCONV_FUSED_GATHER_INTERLEAVE): the grid is cut into
  // units of 8 workgroups (one per XCD); of all_units units, g_units are the
  // gather's, spread evenly among the conv's.  0: the conv's come first.
  int32_t g_interleave;
  uint32_t g_units, all_units;
};

// Request of row t: the last r in [0, n) with off[r] <= t (rows past the
// end clamp to the last request, empty requests never match; r = 0 if
// off[0] > t).  A 64-way search: each round the 64 lanes probe 64 evenly
// spaced offsets of the remaining span, and since the offsets are
// non-decreasing the lanes that see off <= t form a prefix whose length
// (ballot + popcount) names the sub-span to keep.  Two rounds cover 4096
// requests, three cover 262144.  The result is wave-uniform.
__device__ __forceinline__ int32_t find_request(const int32_t* off, int32_t n, int64_t t,
                                                int lane) {
  int32_t base = 0, span = n;
  while (span > 1) {
    const int32_t stride = (span + 63) >> 6;
    const int32_t probe = lane * stride;
    const bool le = probe < span && (int64_t)off[base + (probe < span ? probe : 0)] <= t;
    const int32_t k = (int32_t)__popcll(__ballot(le)) - 1;
    if (k < 0) break;  // off[base] > t: only possible for base 0
    base += k * stride;
    span = (k * stride + stride <= span) ? stride : span - k * stride;
  }
  return uniform(base);
}

__device__ __forceinline__ uint32_t div_magic(uint32_t v, uint32_t magic, uint32_t s1,
                                              uint32_t s2) {
  const uint32_t t = __umulhi(v, magic);
  return (t + ((v - t) >> s1)) >> s2;
}
__device__ __forceinline__ uint32_t div_n(uint32_t v, const FusedParams& p) {
  return div_magic(v, p.n_magic, p.n_s1, p.n_s2);
}

// Build-time tuning knobs (defaults chosen by measurement on MI355X).
#ifndef SCONV_FUSED_BT_MAX
#define SCONV_FUSED_BT_MAX 4       // largest rows-per-wave tile (4, 8 or 16)
#endif
#ifndef SCONV_FUSED_NT_STORES
#define SCONV_FUSED_NT_STORES 1    // streaming (non-temporal) out / cache stores
#endif
#ifndef SCONV_FUSED_NT_OUT
#define SCONV_FUSED_NT_OUT SCONV_FUSED_NT_STORES
#endif
#ifndef SCONV_FUSED_NT_CACHE
#define SCONV_FUSED_NT_CACHE SCONV_FUSED_NT_STORES
#endif
#ifndef SCONV_FUSED_NT_LOADS_MAX_WAVES
#define SCONV_FUSED_NT_LOADS_MAX_WAVES 5120  // streaming x loads up to this many waves
#endif
#ifndef SCONV_FUSED_GROUP_STORES
#define SCONV_FUSED_GROUP_STORES 2  // stores after all rows' arithmetic: 0 never, 1 always,
                                    // 2 in multi-generation launches (no streaming x loads)
#endif
// Launches of several wave generations with multi-row tiles (the prefill)
// reserve LDS they do not use, to hold 4 workgroups per CU instead of the 5
// their registers allow: with the 12 KiB halo buffer 40 KiB of the CU's
// 160 KiB each.  HBM delivers more with fewer bytes in flight per CU
// (0.7-0.8% shorter prefill launches on two boxes; 3 per CU is much slower).
#ifndef SCONV_FUSED_EXTRA_LDS
#define SCONV_FUSED_EXTRA_LDS 28672
#endif
#ifndef SCONV_FUSED_EARLY_INSERT
#define SCONV_FUSED_EARLY_INSERT 1  // cache inserts issued behind the history loads:
                                    // 0 never, 1 one-generation one-stream one-row
                                    // (decode) launches, 2 always
#endif
#ifndef SCONV_FUSED_GATHER_INTERLEAVE
#define SCONV_FUSED_GATHER_INTERLEAVE 0  // combined launch: gather workgroups among the conv's
                                         // (measured slower)
#endif
#ifndef SCONV_FUSED_SERIAL_X
#define SCONV_FUSED_SERIAL_X 0  // one input row in flight per lane (multi-generation launches)
#endif
#ifndef SCONV_FUSED_LDS_WEIGHTS
#define SCONV_FUSED_LDS_WEIGHTS 0  // filter taps shared through LDS by the waves of a workgroup
                                   // (measured slower: the barrier then waits for them too)
#endif
#ifndef SCONV_FUSED_LDS_HALO
#define SCONV_FUSED_LDS_HALO 1  // halo rows passed between the waves of a workgroup
#endif
#ifndef SCONV_FUSED_SLAB_MAJOR
#define SCONV_FUSED_SLAB_MAJOR 1
#endif
#ifndef SCONV_FUSED_XCD_ORDER
#define SCONV_FUSED_XCD_ORDER 1
#endif
#ifndef SCONV_FUSED_XCD_ONE_ROW
#define SCONV_FUSED_XCD_ONE_ROW 0  // XCD runs for one-row slab-major tiles too
#endif
#ifndef SCONV_FUSED_WG_THREADS
#define SCONV_FUSED_WG_THREADS 256
#endif
#ifndef SCONV_FUSED_ENOUGH_WAVES
#define SCONV_FUSED_ENOUGH_WAVES 4096
#endif
#ifndef SCONV_FUSED_NT_HIST
#define SCONV_FUSED_NT_HIST 1  // streaming history loads in one-row tiles with sub-line pieces
#endif
#ifndef SCONV_FUSED_BT_ROW
#define SCONV_FUSED_BT_ROW 1  // one-row tiles of decode-shaped launches guess request t
#endif

#ifndef SCONV_FUSED_MS_ORDER
#define SCONV_FUSED_MS_ORDER 0  // several streams in multi-row tiles: 0 slab-major,
                                // 1 stream-inner, 2 tile-major
#endif
#ifndef SCONV_FUSED_STRIDE
#define SCONV_FUSED_STRIDE 0  // multi-generation one-stream prefill launches in striding waves:
                              // 1 every R-th tile, 2 runs of consecutive tiles (measured slower)
#endif
#ifndef SCONV_FUSED_STRIDE_WAVES
#define SCONV_FUSED_STRIDE_WAVES 4096  // waves of a striding launch (about one per resident slot)
#endif
#ifndef SCONV_FUSED_STRIDE_LDS
#define SCONV_FUSED_STRIDE_LDS 40960  // unused LDS per striding workgroup: 4 workgroups per CU
#endif
#ifndef SCONV_FUSED_DECODE_LANE_BYTES
#define SCONV_FUSED_DECODE_LANE_BYTES 16  // bytes per lane of bf16 one-row tiles: 16, or 8
                                          // (measured slower)
#endif
#ifndef SCONV_FUSED_SMALL_WG_THREADS
#define SCONV_FUSED_SMALL_WG_THREADS 64  // workgroup size of launches below 4096 waves
#endif
#ifndef SCONV_FUSED_BAND_ORDER
#define SCONV_FUSED_BAND_ORDER 0  // multi-generation one-stream launches: 8 bands of rows, one per
                                  // XCD, each walked slab-major
#endif
#ifndef SCONV_FUSED_DECODE_TILE_MAJOR
#define SCONV_FUSED_DECODE_TILE_MAJOR 0  // one stream in one-row tiles: tile-major
#endif

// Wave orders.  Slab-major: consecutive waves walk consecutive tiles of one
// slab.  Tile-major: consecutive waves walk the slabs of one tile.
// Stream-inner (several streams with the same slab count): consecutive
// waves walk the streams of one (slab within stream, tile), then the tiles.
enum { kOrderSlabMajor = 0, kOrderTileMajor = 1, kOrderStreamInner = 2 };
__host__ __device__ constexpr int wave_order(bool multi_stream, int rows_per_tile) {
  return !SCONV_FUSED_SLAB_MAJOR ? kOrderTileMajor
         : (multi_stream && rows_per_tile == 1) ? kOrderTileMajor
         : (multi_stream && SCONV_FUSED_MS_ORDER == 1) ? kOrderStreamInner
         : (multi_stream && SCONV_FUSED_MS_ORDER == 2) ? kOrderTileMajor
         : (!multi_stream && rows_per_tile == 1 && SCONV_FUSED_DECODE_TILE_MAJOR)
             ? kOrderTileMajor
             : kOrderSlabMajor;
}
__host__ __device__ constexpr bool slab_major_order(bool multi_stream, int rows_per_tile) {
  return wave_order(multi_stream, rows_per_tile) == kOrderSlabMajor;
}

// Where a row's request and request start come from (template QM).
constexpr int kQslOff = 0;   // the per-row seq_idx / query_start buffers
constexpr int kQslRegs = 1;  // the offsets qsl, read whole into registers
constexpr int kQslSearch = 2;  // the offsets qsl, searched in device memory
// For launches whose requests have the same small number k of rows (decode:
// k = 1; speculative decode: k = drafts): row t's request is guessed as
// g = t / k and checked against offsets g and g+1, read with the row's
// other metadata; a row that fails the check searches device memory.  One-
// row tiles with k = 1 also read block-table row t at the same time, so a
// row that is request t has its history blocks one dependent round trip
// earlier.
constexpr int kQslGuess = 3;
// Entries of row t read ahead: four 256-byte loads per wave.
constexpr int kBtRowMax = 256;
// Largest rows-per-request count that takes the guess.
constexpr int kGuessMaxRows = 8;
#ifndef SCONV_FUSED_QSL_REG_MAX
#define SCONV_FUSED_QSL_REG_MAX 512
#endif
// Requests that take kQslRegs (at most 512: 8 offsets per lane).
constexpr int kQslRegMax = SCONV_FUSED_QSL_REG_MAX;
static_assert(kQslRegMax <= 512, "8 offsets per lane");

// NTX: input rows loaded as streaming (non-temporal) reads.  MS: several
// streams, each wave finding its own (one-stream launches read entry 0).
// NTH: history rows loaded as streaming reads.
// GW: the launch also runs a window gather in workgroups past the conv's
// (parameters FusedGatherParams).
template <typename D, int VEC, int W, int BT, int QM, bool NTX, bool MS, bool NTH = false,
          bool GW = false>
__global__ __launch_bounds__(SCONV_FUSED_WG_THREADS) void fused_insert_conv_kernel(
    const int64_t* __restrict__ a_positions, const int64_t* __restrict__ a_slot,
    const int32_t* __restrict__ a_qsl, const int32_t* __restrict__ a_bt, int32_t a_T,
    uint32_t a_k_magic, int32_t a_num_reqs, int32_t a_bt_rs, int32_t a_num_slabs,
    uint32_t a_packed, const std::conditional_t<GW, FusedGatherParams, FusedParams> p) {
  // Launch geometry from the leading arguments: tiles, the conv's waves and
  // its workgroups (the host sizes the conv's grid by the same ceiling).
  const uint32_t num_tiles = ((uint32_t)a_T + (uint32_t)(BT - 1)) / (uint32_t)BT;
  const uint32_t wpg_log2 = a_packed >> 20;
  const uint32_t waves_per_group = 1u << wpg_log2;
  // SCONV_FUSED_BAND_ORDER: multi-generation one-stream launches cut the
  // rows into 8 bands of tb tiles (one per XCD, each walked slab-major),
  // with the last band's waves past the rows idle.
  constexpr bool kBand = SCONV_FUSED_BAND_ORDER && BT > 1 && !NTX && !MS && !GW;
  const uint32_t tb = (num_tiles + 7u) / 8u;
  const uint32_t total_waves = kBand ? 8u * tb * (uint32_t)a_num_slabs
                                     : num_tiles * (uint32_t)a_num_slabs;
  const uint32_t num_groups = (total_waves + waves_per_group - 1) >> wpg_log2;
  uint32_t conv_wg = blockIdx.x;  // this workgroup's number among the conv's
  if constexpr (GW) {
    // Gather workgroups come after every conv workgroup, so the hardware
    // hands them out as the conv's resident waves leave room: they fill the
    // conv's latency gaps.  Their inputs are never written by the conv.
    // the gather body's staging, one kGatherLdsWave slice per wave
    __shared__ GatherChunk g_lds[(SCONV_FUSED_WG_THREADS / 64) * kGatherLdsWave];
    constexpr bool kGNt = SCONV_FUSED_GATHER_NT_LOADS;
    bool gather_wg = blockIdx.x >= num_groups;
    uint32_t it = blockIdx.x - num_groups;
    if (SCONV_FUSED_GATHER_INTERLEAVE && p.g_interleave) {
      // Unit u holds gather items g0*8.. (one per lane x of the unit) when
      // the count of gather units up to u grows at u, else conv workgroups
      // (u - g0)*8 + x; both numberings keep x = blockIdx % 8, the XCD.
      const uint32_t u = blockIdx.x >> 3, x = blockIdx.x & 7;
      const uint32_t g0 = (uint32_t)((uint64_t)u * p.g_units / p.all_units);
      const uint32_t g1 = (uint32_t)((uint64_t)(u + 1) * p.g_units / p.all_units);
      gather_wg = g1 > g0;
      it = g0 * 8 + x;
      conv_wg = (u - g1) * 8 + x;
    }
    if (gather_wg) {
      const uint32_t cbs = (uint32_t)p.g.cblocks;
      const int slot = (int)(it / cbs), cb = (int)(it - (it / cbs) * cbs);
      switch (p.g_dc) {
        case 1: gather_window_body<D, VEC, 1, kGNt>(p.g, slot, cb, g_lds); break;
        case 2: gather_window_body<D, VEC, 2, kGNt>(p.g, slot, cb, g_lds); break;
        case 3: gather_window_body<D, VEC, 3, kGNt>(p.g, slot, cb, g_lds); break;
        default: gather_window_body<D, VEC, 4, kGNt>(p.g, slot, cb, g_lds); break;
      }
      return;
    }
  }
  using S = typename D::storage;
  using P = Pack<D, VEC>;
  S* __restrict__ cache = static_cast<S*>(p.cache);
  const int64_t* __restrict__ positions = a_positions;
  const int64_t* __restrict__ slots = a_slot;
  const int32_t* __restrict__ seq_idx = p.seq_idx;
  const int32_t* __restrict__ qstart = p.qs;
  const int32_t* __restrict__ btab = a_bt;
  // The leading arguments (lead_args on the host) arrive preloaded in
  // scalar registers; unpack the packed word.
  const uint32_t k_s1 = a_packed & 1u, k_s2 = (a_packed >> 1) & 31u;
  const int32_t bt_pref = (int32_t)((a_packed >> 8) & 0xfffu);

  // Fields of the parameter block needed to place this wave and to issue
  // its metadata loads (the streams' first slabs, the per-row metadata
  // pointers) all come in the first batch of parameter loads.  A one-stream
  // launch that guesses requests finds everything for its first loads in
  // the leading arguments and waits for the block only behind those loads
  // (below).  A several-stream one waits here for all of it: its waves need
  // the streams' first slabs before they can find their input rows, and
  // waiting behind the first loads added scalar round trips in front of
  // them (a layer's decode step, 5.58-6.05 against 5.36 us).
  constexpr bool kGuess = QM == kQslGuess;
  constexpr bool kPinEarly = !kGuess || MS;
  if constexpr (kPinEarly) {
    asm volatile("" ::"s"(p.seq_idx), "s"(p.qs));
    if constexpr (MS)
      asm volatile("" ::"s"(p.num_streams), "s"(p.st[1].slab0), "s"(p.st[2].slab0),
                   "s"(p.st[3].slab0));
    if constexpr (kGuess)
      asm volatile("" ::"s"(p.n_magic), "s"(p.n_s1), "s"(p.n_s2), "s"(p.N), "s"(p.early_insert),
                   "s"(p.cs0), "s"(p.cs1), "s"(p.cs2), "s"(p.bt_rs));
  }
  constexpr bool kRowAhead = kGuess && BT == 1;  // block-table row read ahead
  constexpr int kOrder = wave_order(MS, BT);
  constexpr bool kSlabMajor = kOrder == kOrderSlabMajor;
  // Workgroups are renumbered so that each XCD runs one contiguous range of
  // waves (neighbouring tiles share halo rows, streams' pieces share cache
  // lines) -- except one-row tiles in slab-major order, where neighbours
  // share nothing and the hardware's round-robin puts the slabs of one row,
  // which read the same block-table row, on the same XCD.
  constexpr bool kXcdRuns = SCONV_FUSED_XCD_ORDER && (BT > 1 || !kSlabMajor || SCONV_FUSED_XCD_ONE_ROW);
  // Stores of multi-row tiles after all rows' arithmetic (in row order)
  // rather than after each row's: measured faster in the many-generation
  // prefill launches, slower in one-generation launches (streaming x loads),
  // where the first row's stores then wait behind every row's history.
  constexpr bool kGroupStores =
      BT > 1 && (SCONV_FUSED_GROUP_STORES == 1 || (SCONV_FUSED_GROUP_STORES == 2 && !NTX));
  const int lane = threadIdx.x & 63;
  // The launch geometry comes from the preloaded leading arguments rather
  // than from the implicit arguments, which would cost a dependent round
  // trip before any data load could start.
  // Wave counts are below 2^31 (checked on the host): 32-bit arithmetic.
  const uint32_t group_wave0 =
      (kXcdRuns ? xcd_contiguous(conv_wg, num_groups) : conv_wg) * waves_per_group;
  uint32_t wave = group_wave0 + (uint32_t)uniform(threadIdx.x >> 6);
  // A wave past the end works on the last tile and writes nothing (no early
  // return: it would split the parameter loads around the branch).
  const bool live_wave = wave < total_waves;
  if (!live_wave) wave = total_waves - 1;
  // Slab-major: consecutive waves walk consecutive tiles of one slab, so
  // the chip advances over rows as one band.  A multi-stream launch of
  // one-row tiles (a layer's decode step) runs tile-major instead: the
  // slabs of all streams for one row are then neighbours on one XCD, and
  // the streams' pieces of a cache row, which share 128-byte lines, meet
  // in one L2.
  uint32_t tile;
  int slab;
  bool band_start = false;  // band order: the slab's first tile in the band
  if constexpr (kBand) {
    const uint32_t per_band = tb * (uint32_t)a_num_slabs;
    const uint32_t band = wave / per_band;
    const uint32_t l = wave - band * per_band;
    const uint32_t slab_u = l / tb;
    tile = band * tb + (l - slab_u * tb);  // past the rows: no row of it is live
    slab = (int)slab_u;
    band_start = l == slab_u * tb;
  } else if constexpr (kSlabMajor) {
    const uint32_t slab_u = wave / num_tiles;
    tile = wave - slab_u * num_tiles;
    slab = (int)slab_u;
  } else if constexpr (kOrder == kOrderStreamInner) {
    // every stream has num_slabs / num_streams slabs (checked on the host)
    const uint32_t S = (uint32_t)p.num_streams;
    const uint32_t rest = wave / S;
    const uint32_t j = rest / num_tiles;
    tile = rest - j * num_tiles;
    slab = (int)((wave - rest * S) * ((uint32_t)a_num_slabs / S) + j);
  } else {
    tile = wave / (uint32_t)a_num_slabs;
    slab = (int)(wave - tile * (uint32_t)a_num_slabs);
  }
  const int64_t t0 = (int64_t)tile * BT;


  // Row metadata of the whole tile in one gather: lane L loads field L % F
  // of row t0 + L / F (position, slot low and high words, and without QSL
  // the request index and request start, or with the request guess the
  // offsets t and t+1), then every value is broadcast to scalar registers.  One instruction cannot be split or sunk below the
  // PAD tests, so the whole tile's metadata costs one round trip.
  // Every load below is unconditional, from an address clamped into the
  // buffers (rows past T, lanes past C): a conditional load would join its
  // value with a default and force an immediate wait for it.
  const int64_t t_last = (int64_t)a_T - 1;
  constexpr int QSL = QM != kQslOff;
  constexpr int F = QSL && !kGuess ? 3 : 5;
  constexpr int NM = F * BT;
  constexpr int NI = (NM + 63) / 64;
  int32_t mv[NI];
#pragma unroll
  for (int g = 0; g < NI; ++g) {
    const int L = g * 64 + lane;
    const int r = L / F;
    const int f = L - r * F;
    const int64_t t = t0 + r < t_last ? t0 + r : t_last;
    const int32_t* src;
    if constexpr (kGuess) {
      // offsets g and g+1 of the row's guessed request (clamped below
      // num_reqs: both exist)
      const int32_t gr = (int32_t)div_magic((uint32_t)t, a_k_magic, k_s1, k_s2);
      const int32_t gq = gr < a_num_reqs - 1 ? gr : a_num_reqs - 1;
      src = f < 3 ? reinterpret_cast<const int32_t*>(f == 0 ? positions : slots) + 2 * t + (f == 2)
                  : a_qsl + gq + (f == 4);
    } else {
      src = f < 3 ? reinterpret_cast<const int32_t*>(f == 0 ? positions : slots) + 2 * t + (f == 2)
                  : (f == 3 ? seq_idx : qstart) + t;
    }
    mv[g] = *src;
  }
  // Up to 512 request offsets: ov[j] of lane L is offset 64*j + L, so each
  // load reads 256 contiguous bytes (indices clamped into the array; the
  // copies past the end are masked below).
  int32_t ov[8];
  if constexpr (QM == kQslRegs) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = j * 64 + lane;
      ov[j] = a_qsl[r < a_num_reqs ? r : a_num_reqs - 1];
    }
  }
  // Block-table row t (the row's guessed request, clamped into the table):
  // entry 64*j + L in brow[j] of lane L, bt_pref entries, clamped.
  int32_t brow[4];
  const int32_t row_guess = (int32_t)(t0 < (int64_t)a_num_reqs - 1 ? t0 : a_num_reqs - 1);
  if constexpr (kRowAhead) {
    const int32_t* row = btab + (int64_t)row_guess * a_bt_rs;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = j * 64 + lane;
      brow[j] = row[e < bt_pref ? e : bt_pref - 1];
    }
  }

  // A one-stream guessing launch has now issued its first loads: the
  // parameter block's fields that the rest of the wave needs are waited for
  // here, in one batch whose loads were issued at the start; fetched at
  // first use, some would add a dependent round trip in front of the
  // history loads.
  if constexpr (kGuess && !kPinEarly) {
    asm volatile("" ::"s"(p.n_magic), "s"(p.n_s1), "s"(p.n_s2), "s"(p.N), "s"(p.early_insert),
                 "s"(p.cs0), "s"(p.cs1), "s"(p.cs2), "s"(p.bt_rs));
    asm volatile("" ::"s"(p.st[0].x), "s"(p.st[0].w), "s"(p.st[0].out), "s"(p.st[0].x_rs),
                 "s"(p.st[0].out_rs), "s"(p.st[0].C), "s"(p.st[0].ws), "s"(p.st[0].off_s),
                 "s"(p.st[0].silu), "s"(p.st[0].residual));
  }

  // The stream owning this slab (its first slab is the last one <= slab).
  // With several streams its fields come with one more scalar load from the
  // parameter segment; the scheduling barrier keeps the metadata loads above
  // issued ahead of it, since their chain (metadata, block table, history)
  // bounds small launches while the stream's fields are needed only for the
  // input rows.  A one-stream launch reads entry 0 at fixed offsets, with
  // the first parameter loads.
  int sid = 0;
  if constexpr (MS) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 1; k < kMaxStreams; ++k)
      sid = (k < p.num_streams && slab >= p.st[k].slab0) ? k : sid;
  }
  const S* x;
  const S* wt;
  S* out;
  int64_t x_rs, out_rs, w_sc, w_sk;
  int32_t s_C, s_ws, s_off, s_silu, s_res, s_slab0;
  auto take = [&](const FusedStream& fs) {
    x = static_cast<const S*>(fs.x);
    wt = static_cast<const S*>(fs.w);
    out = static_cast<S*>(fs.out);
    x_rs = fs.x_rs; out_rs = fs.out_rs; w_sc = fs.w_sc; w_sk = fs.w_sk;
    s_C = fs.C; s_ws = fs.ws; s_off = fs.off_s; s_silu = fs.silu; s_res = fs.residual;
    s_slab0 = fs.slab0;
  };
  if constexpr (MS) take(p.st[uniform(sid)]);
  else take(p.st[0]);
  const int lslab = slab - s_slab0;  // slab within the stream

  // The tile's input rows (16 bytes per lane).
  const int c0 = (lslab * 64 + lane) * VEC;  // lane's channels lie in one head
  const bool on = c0 < s_C;
  const int cl = on ? c0 : 0;               // clamped for the loads
  P xr[BT];
  // SCONV_FUSED_SERIAL_X: in launches of several wave generations, each row
  // is loaded only once the previous one has arrived (its address takes a
  // zero computed from that row's data), so a lane has one input row in
  // flight at a time rather than the whole tile.
  constexpr bool kSerialX = SCONV_FUSED_SERIAL_X && !NTX && BT > 1 && VEC > 1;
  int32_t dep = 0;
#pragma unroll
  for (int i = 0; i < BT; ++i) {
    const int64_t t = t0 + i < t_last ? t0 + i : t_last;
    if constexpr (NTX) xr[i].load_nt(x + t * x_rs + cl);
    else xr[i].load(x + t * x_rs + cl + dep);
    if constexpr (kSerialX) {
      if (i + 1 < BT) asm volatile("v_mov_b32 %0, 0" : "=v"(dep) : "v"(xr[i].raw[0]));
    }
  }
  const int h = on ? c0 / s_ws : 0;
  const int j = c0 - h * s_ws;
  const int64_t lane_off = (int64_t)h * p.cs1 + s_off + j;

  // Filter taps of this lane's channels, as raw elements [e][k]; widened to
  // fp32 after the metadata is in.  The 16-byte-lane kernels take packed
  // [C, W] weights (VEC*W consecutive elements per lane, moved as 16-byte
  // chunks); the one-channel kernels read any strides.
  constexpr int kChunk = 16 / (int)sizeof(S);
  constexpr int kN = VEC * W;
  constexpr int kNChunks = kN / kChunk > 0 ? kN / kChunk : 1;
  Pack<D, kChunk> wpk[kNChunks];
  struct WRaw { S e[kN]; } wr;
  // Launches of several wave generations in slab-major order hand halo rows
  // between the waves of a workgroup through LDS, behind one barrier (see
  // the halo below).  The same barrier lets waves that work on one slab
  // share its filter taps: wave w loads chunks w, w + waves, ... for all
  // 64 lanes and leaves them in LDS, so each wave issues one load for its
  // taps instead of kNChunks.  Whether every wave of the workgroup is on
  // one slab is the same test in each of them (first and last wave).
#if SCONV_FUSED_LDS_HALO
  constexpr bool kLdsHalo = kSlabMajor && !NTX && W > 1 && BT >= W - 1;
#else
  constexpr bool kLdsHalo = false;
#endif
  constexpr bool kLdsWts = kLdsHalo && VEC > 1 && SCONV_FUSED_LDS_WEIGHTS;
  const int wpg = (int)waves_per_group;
  const int wig = (int)(threadIdx.x >> 6);  // wave in workgroup
  bool wts_shared = false;
  if constexpr (kLdsWts) {
    const uint32_t last = total_waves - 1;
    const uint32_t wa = group_wave0 < last ? group_wave0 : last;
    const uint32_t wb = group_wave0 + (uint32_t)wpg - 1 < last ? group_wave0 + (uint32_t)wpg - 1 : last;
    wts_shared = wa / num_tiles == wb / num_tiles;
  }
  if constexpr (VEC > 1) {
    static_assert(kN % kChunk == 0, "packed weights come in whole 16-byte chunks");
    if (wts_shared) {
#pragma unroll
      for (int ch = 0; ch < kNChunks; ++ch)
        if (ch % wpg == wig) wpk[ch].load(wt + (int64_t)cl * W + ch * kChunk);
    } else {
#pragma unroll
      for (int ch = 0; ch < kNChunks; ++ch) wpk[ch].load(wt + (int64_t)cl * W + ch * kChunk);
    }
  } else {
#pragma unroll
    for (int k = 0; k < W; ++k) wr.e[k] = wt[(int64_t)cl * w_sc + (int64_t)k * w_sk];
  }

  // The parameters needed from here on (addressing, epilogue flags) must
  // arrive while the loads above are in flight; fetched at first use they
  // would add a dependent round trip after the metadata returns.  An empty
  // statement taking them as scalar inputs pins their loads here.
  asm volatile("" ::"s"(p.n_magic), "s"(p.n_s1), "s"(p.n_s2), "s"(p.N), "s"(p.early_insert),
               "s"(s_silu), "s"(s_res), "s"(p.cs0), "s"(p.cs2), "s"(p.bt_rs),
               "s"(out_rs));

  // Broadcast the metadata.  Positions and slots are below max_blocks*N and
  // num_blocks*N, both checked on the host to fit in 31 bits; a negative
  // 64-bit slot is PAD, and so is every row of a wave past the end.
  int32_t pos[BT], slot[BT], req[BT], qs[BT];
#pragma unroll
  for (int i = 0; i < BT; ++i) {
    const int b = F * i;
    pos[i] = __builtin_amdgcn_readlane(mv[b / 64], b % 64);
    const int32_t lo = __builtin_amdgcn_readlane(mv[(b + 1) / 64], (b + 1) % 64);
    const int32_t hi = __builtin_amdgcn_readlane(mv[(b + 2) / 64], (b + 2) % 64);
    slot[i] = (hi < 0 || !live_wave || t0 + i > t_last) ? -1 : lo;
    if constexpr (!QSL || kGuess) {
      req[i] = __builtin_amdgcn_readlane(mv[(b + 3) / 64], (b + 3) % 64);
      qs[i] = __builtin_amdgcn_readlane(mv[(b + 4) / 64], (b + 4) % 64);
    } else {
      req[i] = 0;
      qs[i] = 0;
    }
  }
  if constexpr (kGuess) {
    // req / qs hold offsets g and g+1 of each row's guess g.  Row t lies in
    // request g exactly when off[g] <= t < off[g+1] (offsets are non-
    // decreasing, so no later request starts at or before t); otherwise
    // (empty or longer requests before it, rows past the last offset) a
    // live row searches device memory.
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      const int32_t t = (int32_t)(t0 + i < t_last ? t0 + i : t_last);
      const int32_t g = (int32_t)div_magic((uint32_t)t, a_k_magic, k_s1, k_s2);
      const int32_t gq = g < a_num_reqs - 1 ? g : a_num_reqs - 1;
      const int32_t lo = req[i], hi = qs[i];
      if (lo <= t && t < hi) {
        req[i] = gq;
        qs[i] = lo;
      } else if (slot[i] >= 0) {
        req[i] = find_request(a_qsl, a_num_reqs, t, lane);
        qs[i] = uniform(a_qsl[req[i]]);
      } else {
        req[i] = 0;
        qs[i] = 0;
      }
    }
  }
  if constexpr (QM == kQslRegs) {
    // Offsets in registers: the count of offsets <= t is t's request plus
    // one (offsets are non-decreasing; those past the end are masked to
    // INT32_MAX), summed over the eight 64-offset runs by ballot and
    // popcount.  A tile whose first and last rows count the same lies in
    // one request.
#pragma unroll
    for (int run = 0; run < 8; ++run)
      if (run * 64 + lane >= a_num_reqs) ov[run] = INT32_MAX;
    auto count_le = [&](int32_t row) -> int32_t {
      int32_t c = 0;
#pragma unroll
      for (int run = 0; run < 8; ++run) c += (int32_t)__popcll(__ballot(ov[run] <= row));
      return c;
    };
    auto offset_of = [&](int32_t r) -> int32_t {
      const int32_t l = r & 63, run = r >> 6;
      int32_t v = __builtin_amdgcn_readlane(ov[0], l);
#pragma unroll
      for (int q = 1; q < 8; ++q) {
        const int32_t vq = __builtin_amdgcn_readlane(ov[q], l);
        v = run == q ? vq : v;
      }
      return v;
    };
    const int32_t tl = (int32_t)t_last;
    const int32_t ta = t0 < tl ? (int32_t)t0 : tl;
    const int32_t ca = count_le(ta);
    int32_t cb = ca;
    if constexpr (BT > 1) {
      const int32_t tb = t0 + BT - 1 < tl ? (int32_t)(t0 + BT - 1) : tl;
      cb = count_le(tb);
    }
    if (ca == cb) {
      const int32_t r = ca > 0 ? ca - 1 : 0;  // rows before the first offset: request 0
      const int32_t q = offset_of(r);
#pragma unroll
      for (int i = 0; i < BT; ++i) {
        req[i] = r;
        qs[i] = q;
      }
    } else {
#pragma unroll
      for (int i = 0; i < BT; ++i) {
        const int32_t t = t0 + i < tl ? (int32_t)(t0 + i) : tl;
        const int32_t c = count_le(t);
        req[i] = c > 0 ? c - 1 : 0;
        qs[i] = offset_of(req[i]);
      }
    }
  }
  if constexpr (QM == kQslSearch) {
    // More requests than fit in registers: each wave searches device memory
    // for the request r0 of its first row, reads the 64 offsets from r0 on
    // in one access, and every row's request is r0 plus the count of those
    // offsets <= row, less one.  Only when 64 request starts fall inside one
    // tile (empty requests) can a row lie past that window; such a row
    // searches on its own.  (Staging the offsets in LDS per workgroup was
    // measured slower: it moves every offset to every workgroup.)
    const int32_t n = a_num_reqs;
    const int64_t tf = t0 < t_last ? t0 : t_last;
    const int32_t r0 = find_request(a_qsl, n, tf, lane);
    const int32_t wnd = a_qsl[r0 + lane < n ? r0 + lane : n - 1];
    const bool in_window = lane < n - r0;
    const bool beyond = r0 + 64 < n;
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      const int64_t t = t0 + i;
      int32_t k = (int32_t)__popcll(__ballot(in_window && (int64_t)wnd <= t)) - 1;
      k = k < 0 ? 0 : k;  // rows before the first offset belong to request 0
      req[i] = r0 + k;
      qs[i] = __builtin_amdgcn_readlane(wnd, k);
      if (k == 63 && beyond && slot[i] >= 0) {
        req[i] = find_request(a_qsl, n, t, lane);
        qs[i] = uniform(a_qsl[req[i]]);
      }
    }
  }

  // Halo: input rows t0-m (m = 1..W-1) that a row of this tile reads as a
  // same-forward tap.
  constexpr int kHalo = W > 1 ? W - 1 : 1;
  P halo[kHalo];
  // In slab-major order the waves of a workgroup hold consecutive tiles of
  // one slab, so a wave's halo rows are the previous wave's last rows:
  // each wave leaves its last W-1 rows in LDS and, after one barrier, the
  // next wave takes them from there instead of reading them again through
  // L2.  The first wave of a workgroup, and a wave whose tile is the first
  // of its slab, still load their halo.  Only launches of several wave
  // generations do this: when all waves are resident at once, the barrier
  // would hold back the history lookups that bound such launches.
  constexpr int kWavesMax = SCONV_FUSED_WG_THREADS / 64;
  __shared__ typename P::raw_t s_halo[kLdsHalo ? kWavesMax : 1][kHalo][64];
  __shared__ typename Pack<D, kChunk>::raw_t s_wts[kLdsWts ? kNChunks : 1][64];
  bool halo_from_lds = false;
  if constexpr (kLdsHalo) {
#pragma unroll
    for (int m = 1; m <= W - 1; ++m) s_halo[wig][m - 1][lane] = xr[BT - m].raw;
    if constexpr (kLdsWts) {
      if (wts_shared) {
#pragma unroll
        for (int ch = 0; ch < kNChunks; ++ch)
          if (ch % wpg == wig) s_wts[ch][lane] = wpk[ch].raw;
      }
    }
    __syncthreads();
    if constexpr (kLdsWts) {
      if (wts_shared) {
#pragma unroll
        for (int ch = 0; ch < kNChunks; ++ch) wpk[ch].raw = s_wts[ch][lane];
      }
    }
    // (a slab's first tile takes no halo from the previous wave, which
    // holds another slab's tile)
    halo_from_lds = wig > 0 && (kBand ? !band_start : tile > 0);
  }
  if (halo_from_lds) {
#pragma unroll
    for (int m = 1; m <= W - 1; ++m) halo[m - 1].raw = s_halo[kLdsHalo ? wig - 1 : 0][m - 1][lane];
  } else {
#pragma unroll
    for (int m = 1; m <= kHalo; ++m) {
      bool need = false;
      if (m <= W - 1) {
#pragma unroll
        for (int i = 0; i < BT && i <= W - 1 - m; ++i)
          need |= slot[i] >= 0 && pos[i] - (i + m) >= 0 && t0 - m >= (int64_t)qs[i] && t0 - m >= 0;
      }
      // Loaded only where read (the tap choice below reads halo m exactly
      // for the rows counted in `need`), and left unset otherwise: merging
      // with a default value would make the wave wait for the load right
      // here, in front of the history lookups.
      if (need && on) halo[m - 1].load(x + (t0 - m) * x_rs + c0);
    }
  }


  // Stores of row i (lanes past C store nothing): its output and its input
  // row into the cache slot.
  P outv[BT];
  // The insert of row i: its input row into its cache slot.
  auto insert_row = [&](int i) {
    const uint32_t blk = div_n((uint32_t)slot[i], p);
    const int32_t off = slot[i] - (int32_t)blk * p.N;
#if SCONV_FUSED_NT_CACHE
    xr[i].store_nt(cache + (int64_t)blk * p.cs0 + (int64_t)off * p.cs2 + lane_off);
#else
    xr[i].store(cache + (int64_t)blk * p.cs0 + (int64_t)off * p.cs2 + lane_off);
#endif
  };
  // A decode wave's stores would otherwise all start after its history
  // arrives; the insert needs only the slot and the input row, so it is
  // issued as soon as the history loads are, and overlaps that round trip.
  // No slot written by a call is a pre-forward tap of the same call (the
  // caller's contract), so an early insert cannot change what the history
  // loads read.  In larger one-generation launches (speculative decode, a
  // layer's four streams) the early stores slow the history loads they
  // travel with, and measured slower.
  constexpr bool kEarlyInsert =
      SCONV_FUSED_EARLY_INSERT == 2 || (SCONV_FUSED_EARLY_INSERT == 1 && NTH && !MS);
  const bool early = kEarlyInsert && p.early_insert;  // the host's choice, per launch
  auto store_row = [&](int i) {
    if (on) {
      const int64_t t = t0 + i;
#if SCONV_FUSED_NT_OUT
      outv[i].store_nt(out + t * out_rs + c0);
#else
      outv[i].store(out + t * out_rs + c0);
#endif
      if (!early) insert_row(i);
    }
  };
  // Output of row i from its fp32 accumulators: SiLU, residual, round.
  auto finish = [&](int i, const float (&acc)[VEC]) {
    float y[VEC];
    {
      float cur[VEC];
      xr[i].to_float(cur);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float v = acc[e];
        if (s_silu) v = silu(v);
        if (s_res) v += cur[e];
        y[e] = v;
      }
    }
    outv[i].from_float(y);
    if constexpr (!kGroupStores) store_row(i);
  };


  // History rows 1..W-1 of the current request, in named registers (an
  // array indexed by a run-time value would be demoted to LDS).
  P hist1, hist2, hist3;
  hist1.zero();
  hist2.zero();
  hist3.zero();
  int32_t hist_req = -1;  // request whose history rows are held
  float wk[W][VEC];        // filter taps in fp32, widened after row 0's history fetch
#pragma unroll
  for (int i = 0; i < BT; ++i) {
    const int64_t t = t0 + i;

    // Pre-forward taps of a row are its request's history: the cache rows
    // at positions first-1 .. first-(W-1), first = the request's first
    // position in this call.  Rows of one request share them, so they are
    // fetched once, by the request's first row in the tile (the one that
    // needs the most of them), and kept in registers for the others.
    const int32_t d = (int32_t)(t - qs[i]);  // row offset inside its request
    if (slot[i] >= 0 && d < W - 1 && req[i] != hist_req && pos[i] - d > 0) {
      // first > 0, so history row 1 (position first-1) is read by this row
      // and its block-table entry is valid.  The history loads below are
      // unconditional (a load inside a branch would wait for its value at
      // the join): rows this request does not read, m > W-1-d or before
      // position 0, are fetched from history row 1's address instead.  The
      // block-table entries come from registers or from one uniform branch
      // of lookups, whose values the history addresses need at once anyway.
      const int32_t first = pos[i] - d;
      // Entries read lie in [0, num_blocks): unsigned, so widening one for
      // the address does not wait on its load the way sign-extension does.
      uint32_t hblk[kHalo];
      int32_t hoff[kHalo];
      uint32_t hlb[kHalo];
#pragma unroll
      for (int m = 1; m <= W - 1; ++m) {
        const int32_t src = first - m >= 0 ? first - m : 0;
        hlb[m - 1] = div_n((uint32_t)src, p);
        hoff[m - 1] = src - (int32_t)hlb[m - 1] * p.N;
      }
      // A row this request does not read takes history row 1's place.
#pragma unroll
      for (int m = 2; m <= W - 1; ++m) {
        if (!(m <= W - 1 - d && first - m >= 0)) {
          hlb[m - 1] = hlb[0];
          hoff[m - 1] = hoff[0];
        }
      }
      // History row 1 has the largest block index of the W-1.
      bool in_regs = false;
      if constexpr (kRowAhead) in_regs = req[i] == row_guess && hlb[0] < (uint32_t)bt_pref;
      if (in_regs) {
#pragma unroll
        for (int m = 1; m <= W - 1; ++m) {
          const int32_t l = (int32_t)(hlb[m - 1] & 63), q = (int32_t)(hlb[m - 1] >> 6);
          int32_t v = __builtin_amdgcn_readlane(brow[0], l);
#pragma unroll
          for (int jj = 1; jj < 4; ++jj) {
            const int32_t vj = __builtin_amdgcn_readlane(brow[jj], l);
            v = q == jj ? vj : v;
          }
          hblk[m - 1] = (uint32_t)v;
        }
      } else {
        // Scalar loads (the table is read-only for the launch): their wait
        // counts apart from the vector loads in flight, so the history
        // loads need not wait for the tile's input rows to land.
        const __attribute__((address_space(4))) int32_t* bt_c =
            (const __attribute__((address_space(4))) int32_t*)btab;
#pragma unroll
        for (int m = 1; m <= W - 1; ++m)
          hblk[m - 1] = (uint32_t)bt_c[(int64_t)req[i] * p.bt_rs + hlb[m - 1]];
        // All lookups in flight before any of them is used (the scheduler
        // would otherwise start on the first one's address arithmetic and
        // wait for it before issuing the next).
        __builtin_amdgcn_sched_barrier(0);
      }
      auto fetch = [&](int m, P& dst) {
        const S* src = cache + (int64_t)hblk[m - 1] * p.cs0 + (int64_t)hoff[m - 1] * p.cs2 + (on ? lane_off : 0);
        if constexpr (NTH) dst.load_nt(src);
        else dst.load(src);
      };
      if constexpr (W > 1) fetch(1, hist1);
      if constexpr (W > 2) fetch(2, hist2);
      if constexpr (W > 3) fetch(3, hist3);
      hist_req = req[i];
    }
    if constexpr (kEarlyInsert) {
      if (early && i == 0 && on) {
#pragma unroll
        for (int r = 0; r < BT; ++r)
          if (slot[r] >= 0) insert_row(r);
      }
    }
    // Widening here rather than before the loop keeps the wait for the
    // weights (which, counted in order, also waits for the halo loads)
    // behind the issue of the history lookups.
    if (i == 0) {
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int k = 0; k < W; ++k) {
          if constexpr (VEC > 1) {
            const int flat = e * W + k;
            wk[k][e] = to_float<D>(__builtin_bit_cast(typename Pack<D, kChunk>::Elems,
                                                      wpk[flat / kChunk].raw).e[flat % kChunk]);
          } else {
            wk[k][e] = to_float<D>(wr.e[k]);
          }
        }
    }
    if (slot[i] < 0) continue;  // PAD (or past T): no output, no insert

    // Taps, oldest first: pick the raw 16 bytes (uniform choice), widen,
    // accumulate in fp32.
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const int lag = W - 1 - k;
      P src;
      if (lag == 0) {
        src = xr[i];
      } else if (pos[i] - lag < 0) {
        src.zero();                                   // before position 0
      } else if (lag <= d) {
        src = i >= lag ? xr[i >= lag ? i - lag : 0]   // same forward: x row t-lag
                       : halo[lag - i - 1 >= 0 ? lag - i - 1 : 0];
      } else {
        const int m = lag - d;                        // before this forward
        if (m == 1) src = hist1;
        else if (m == 2) src = hist2;
        else src = hist3;
      }
      float f[VEC];
      src.to_float(f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = __builtin_fmaf(wk[k][e], f[e], acc[e]);
    }
    finish(i, acc);
  }
  if constexpr (kGroupStores) {
#pragma unroll
    for (int i = 0; i < BT; ++i)
      if (slot[i] >= 0) store_row(i);
  }
}

#if SCONV_FUSED_STRIDE
// ---------------------------------------------------------------- striding waves
//
// A measured alternative for the multi-generation prefill shape (one
// stream, per-row request buffers, 16-byte lanes, four-row tiles), built
// only with SCONV_FUSED_STRIDE: about one wave per resident slot, each
// taking many tiles of one slab (every R-th tile, or a run of consecutive
// ones) with its filter taps loaded once.  Each tile's halo rows come with
// its input rows.  Stores are buffer stores issued for every row and lane,
// a PAD row's or an idle lane's with an offset past the buffer's range
// (dropped by the hardware), so that the number of stores per tile is
// fixed and a wait for the next tile's loads never waits for them.  Per
// row it computes what fused_insert_conv_kernel computes.  Both orders
// measured slower than one-tile waves.
constexpr int32_t kDropOffset = (int32_t)0x80000000;
constexpr int32_t kRangeBytes = 0x7ffffff0;

template <typename D, int VEC, int W>
__global__ __launch_bounds__(SCONV_FUSED_WG_THREADS) void fused_stride_kernel(const FusedParams p) {
  using S = typename D::storage;
  using P = Pack<D, VEC>;
  static_assert(sizeof(typename P::raw_t) == 16, "16-byte lanes");
  constexpr int BT = 4;
  constexpr int F = 5;
  constexpr int kHalo = W > 1 ? W - 1 : 1;
  S* __restrict__ cache = static_cast<S*>(p.cache);
  const S* __restrict__ x = static_cast<const S*>(p.st[0].x);
  const S* __restrict__ wt = static_cast<const S*>(p.st[0].w);
  S* __restrict__ out = static_cast<S*>(p.st[0].out);
  const int64_t x_rs = p.st[0].x_rs, out_rs = p.st[0].out_rs;
  const int lane = threadIdx.x & 63;
  const uint32_t per_slab = (uint32_t)p.walk_per_slab;
  const uint32_t num_tiles = (uint32_t)p.num_tiles;
  const uint32_t wave = xcd_contiguous(blockIdx.x, p.num_groups) * (uint32_t)p.waves_per_group +
                        (uint32_t)uniform(threadIdx.x >> 6);
  if (wave >= per_slab * (uint32_t)p.num_slabs) return;
  const uint32_t slab = wave / per_slab;
  const uint32_t r0 = wave - slab * per_slab;
  if (r0 >= num_tiles) return;
  const int c0 = ((int)slab * 64 + lane) * VEC;
  const bool on = c0 < p.st[0].C;
  const int cl = on ? c0 : 0;
  const int h = on ? c0 / p.st[0].ws : 0;
  const int jc = c0 - h * p.st[0].ws;
  const int64_t lane_off = (int64_t)h * p.cs1 + p.st[0].off_s + jc;
  const int64_t t_last = p.T - 1;
  const int32_t* __restrict__ seq_idx = p.seq_idx;
  const int32_t* __restrict__ qstart = p.qs;
  const int64_t* __restrict__ positions = p.positions;
  const int64_t* __restrict__ slots = p.slot;
  const int32_t* __restrict__ btab = p.bt;
  const bool s_silu = p.st[0].silu != 0, s_res = p.st[0].residual != 0;
  constexpr int kAux = SCONV_FUSED_NT_STORES ? 2 : 0;
  auto load_tile = [&](uint32_t tile, int32_t& mv, P (&xr)[BT], P (&hl)[kHalo]) {
    const int64_t t0 = (int64_t)tile * BT;
    const int r = lane / F, f = lane - (lane / F) * F;
    const int64_t t = t0 + r < t_last ? t0 + r : t_last;
    const int32_t* src =
        f < 3 ? reinterpret_cast<const int32_t*>(f == 0 ? positions : slots) + 2 * t + (f == 2)
              : (f == 3 ? seq_idx : qstart) + t;
    mv = *src;
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      const int64_t ti = t0 + i < t_last ? t0 + i : t_last;
      xr[i].load(x + ti * x_rs + cl);
    }
#pragma unroll
    for (int m = 1; m <= kHalo; ++m) {
      const int64_t th = t0 - m >= 0 ? t0 - m : 0;
      hl[m - 1].load(x + th * x_rs + cl);
    }
  };
  constexpr int kChunk = 16 / (int)sizeof(S);
  constexpr int kN = VEC * W;
  static_assert(kN % kChunk == 0, "packed weights come in whole 16-byte chunks");
  constexpr int kNChunks = kN / kChunk;
  Pack<D, kChunk> wpk[kNChunks];
#pragma unroll
  for (int ch = 0; ch < kNChunks; ++ch) wpk[ch].load(wt + (int64_t)cl * W + ch * kChunk);
  auto wk = [&](int k, int e) -> float {
    const int flat = e * W + k;
    return to_float<D>(__builtin_bit_cast(typename Pack<D, kChunk>::Elems,
                                          wpk[flat / kChunk].raw).e[flat % kChunk]);
  };
  auto process = [&](uint32_t tile, const int32_t mv, const P (&xr)[BT], const P (&halo)[kHalo],
                     auto&& between) {
    const int64_t t0 = (int64_t)tile * BT;
#pragma unroll
    for (int ch = 0; ch < kNChunks; ++ch) asm volatile("" : "+v"(wpk[ch].raw));
    int32_t pos[BT], slot[BT], req[BT], qs[BT];
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      pos[i] = __builtin_amdgcn_readlane(mv, F * i);
      const int32_t lo = __builtin_amdgcn_readlane(mv, F * i + 1);
      const int32_t hi = __builtin_amdgcn_readlane(mv, F * i + 2);
      slot[i] = (hi < 0 || t0 + i > t_last) ? -1 : lo;
      req[i] = __builtin_amdgcn_readlane(mv, F * i + 3);
      qs[i] = __builtin_amdgcn_readlane(mv, F * i + 4);
    }
    P hist1, hist2, hist3;
    hist1.zero();
    hist2.zero();
    hist3.zero();
    int32_t hist_req = -1;
    P outv[BT];
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      outv[i].zero();
      const int64_t t = t0 + i;
      const int32_t d = (int32_t)(t - qs[i]);
      if (slot[i] >= 0 && d < W - 1 && req[i] != hist_req && pos[i] - d > 0) {
        const int32_t first = pos[i] - d;
        uint32_t hblk[kHalo];
        int32_t hoff[kHalo];
        uint32_t hlb[kHalo];
#pragma unroll
        for (int m = 1; m <= W - 1; ++m) {
          const int32_t src = first - m >= 0 ? first - m : 0;
          hlb[m - 1] = div_n((uint32_t)src, p);
          hoff[m - 1] = src - (int32_t)hlb[m - 1] * p.N;
        }
#pragma unroll
        for (int m = 2; m <= W - 1; ++m) {
          if (!(m <= W - 1 - d && first - m >= 0)) {
            hlb[m - 1] = hlb[0];
            hoff[m - 1] = hoff[0];
          }
        }
        const __attribute__((address_space(4))) int32_t* bt_c =
            (const __attribute__((address_space(4))) int32_t*)btab;
#pragma unroll
        for (int m = 1; m <= W - 1; ++m)
          hblk[m - 1] = (uint32_t)bt_c[(int64_t)req[i] * p.bt_rs + hlb[m - 1]];
        __builtin_amdgcn_sched_barrier(0);
        auto fetch = [&](int m, P& dst) {
          dst.load(cache + (int64_t)hblk[m - 1] * p.cs0 + (int64_t)hoff[m - 1] * p.cs2 +
                   (on ? lane_off : 0));
        };
        if constexpr (W > 1) fetch(1, hist1);
        if constexpr (W > 2) fetch(2, hist2);
        if constexpr (W > 3) fetch(3, hist3);
        hist_req = req[i];
      }
      if (slot[i] < 0) continue;
      float acc[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const int lag = W - 1 - k;
        P src;
        if (lag == 0) {
          src = xr[i];
        } else if (pos[i] - lag < 0) {
          src.zero();
        } else if (lag <= d) {
          src = i >= lag ? xr[i >= lag ? i - lag : 0] : halo[lag - i - 1 >= 0 ? lag - i - 1 : 0];
        } else {
          const int m = lag - d;
          if (m == 1) src = hist1;
          else if (m == 2) src = hist2;
          else src = hist3;
        }
        float f[VEC];
        src.to_float(f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = __builtin_fmaf(wk(k, e), f[e], acc[e]);
      }
      float y[VEC];
      {
        float cur[VEC];
        xr[i].to_float(cur);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float v = acc[e];
          if (s_silu) v = silu(v);
          if (s_res) v += cur[e];
          y[e] = v;
        }
      }
      outv[i].from_float(y);
    }
    between();
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      const bool live = slot[i] >= 0;
      const int64_t t = live ? t0 + i : 0;
      const __amdgpu_buffer_rsrc_t ro =
          __builtin_amdgcn_make_buffer_rsrc(out + t * out_rs, 0, kRangeBytes, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b128(
          outv[i].raw, ro, live && on ? c0 * (int32_t)sizeof(S) : kDropOffset, 0, kAux);
      const uint32_t blk = live ? div_n((uint32_t)slot[i], p) : 0u;
      const int32_t off = live ? slot[i] - (int32_t)blk * p.N : 0;
      const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
          cache + (int64_t)blk * p.cs0 + (int64_t)off * p.cs2, 0, kRangeBytes, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b128(
          xr[i].raw, rc, live && on ? (int32_t)(lane_off * (int64_t)sizeof(S)) : kDropOffset, 0,
          kAux);
    }
  };
  // Mode 1: wave r takes tiles r, r + R, r + 2R, ... (the chip works on
  // one band of R tiles at a time).  Mode 2: wave r takes the run of
  // ceil(tiles / R) consecutive tiles starting at r times that.
  const uint32_t R = per_slab;
  uint32_t first, step, end;
  if constexpr (SCONV_FUSED_STRIDE == 2) {
    const uint32_t L = (num_tiles + R - 1) / R;
    first = r0 * L;
    step = 1;
    end = first + L < num_tiles ? first + L : num_tiles;
    if (first >= end) return;
  } else {
    first = r0;
    step = R;
    end = num_tiles;
  }
  // Two register sets in turn; a tile's successor is loaded between its
  // arithmetic and its stores (the last tile reloads its own rows); the
  // first two tiles run ahead of the loop, so that every path into it has
  // the same loads and stores outstanding.
  int32_t mv_a, mv_b;
  P xr_a[BT], xr_b[BT], hl_a[kHalo], hl_b[kHalo];
  auto nxt = [&](uint32_t t) { return t + step < end ? t + step : t; };
  uint32_t tile = first;
  load_tile(tile, mv_a, xr_a, hl_a);
  process(tile, mv_a, xr_a, hl_a, [&] { load_tile(nxt(tile), mv_b, xr_b, hl_b); });
  if (tile + step >= end) return;
  process(tile + step, mv_b, xr_b, hl_b, [&] { load_tile(nxt(tile + step), mv_a, xr_a, hl_a); });
  for (tile += 2 * step; tile < end; tile += 2 * step) {
    process(tile, mv_a, xr_a, hl_a, [&] { load_tile(nxt(tile), mv_b, xr_b, hl_b); });
    if (tile + step >= end) break;
    process(tile + step, mv_b, xr_b, hl_b, [&] { load_tile(nxt(tile + step), mv_a, xr_a, hl_a); });
  }
}

template <typename D, int VEC>
static void launch_stride(int W, const FusedParams& p, uint32_t g, uint32_t th, hipStream_t s) {
  constexpr uint32_t kLds = SCONV_FUSED_STRIDE_LDS;
  switch (W) {
    case 1: hipLaunchKernelGGL((fused_stride_kernel<D, VEC, 1>), dim3(g), dim3(th), kLds, s, p); break;
    case 2: hipLaunchKernelGGL((fused_stride_kernel<D, VEC, 2>), dim3(g), dim3(th), kLds, s, p); break;
    case 3: hipLaunchKernelGGL((fused_stride_kernel<D, VEC, 3>), dim3(g), dim3(th), kLds, s, p); break;
    default: hipLaunchKernelGGL((fused_stride_kernel<D, VEC, 4>), dim3(g), dim3(th), kLds, s, p); break;
  }
}
#endif

// ---------------------------------------------------------------- dispatch

// A fused launch passes, ahead of its parameter block, the values every
// wave needs before its first memory access as leading scalar arguments
// (the kernel's a_* arguments; an aggregate argument is never preloaded):
// the build has the compiler ask the hardware to preload the first 14
// dwords of the argument segment into scalar registers
// (-amdgpu-kernarg-preload-count), which takes the round trip of a first
// parameter load off the front of a decode launch's dependent chain.
// Packed word: bit 0 k_s1, bits 1-5 k_s2, bits 8-19 bt_pref, bits 20-31
// log2 of the waves per workgroup (the host keeps each field in range).
static_assert((SCONV_FUSED_WG_THREADS & (SCONV_FUSED_WG_THREADS - 1)) == 0,
              "workgroups of a power-of-two number of waves");
template <typename Kern, typename Prm>
static void launch_fused(Kern kern, uint32_t grid, uint32_t threads, uint32_t lds, hipStream_t s,
                         const Prm& p) {
  const uint32_t packed = (p.k_s1 & 1u) | ((p.k_s2 & 31u) << 1) | ((uint32_t)p.bt_pref << 8) |
                          ((uint32_t)__builtin_ctz((uint32_t)p.waves_per_group) << 20);
  const int32_t bt_rs = p.bt_rs <= INT32_MAX ? (int32_t)p.bt_rs : 0;  // read ahead only below
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, s, p.positions, p.slot, p.qsl, p.bt,
                     (int32_t)p.T, p.k_magic, p.num_reqs, bt_rs, p.num_slabs, packed, p);
}

template <typename D, int VEC, int W, int BT, bool NTX, bool MS, bool NTH = false>
static void launch_q(const FusedParams& p, uint32_t grid, uint32_t threads, hipStream_t s) {
  constexpr uint32_t kExtraLds = NTX || BT == 1 ? 0u : (uint32_t)SCONV_FUSED_EXTRA_LDS;
  if constexpr (W > 1) {
    if (p.guess) {
      launch_fused(fused_insert_conv_kernel<D, VEC, W, BT, kQslGuess, NTX, MS, NTH>,
                 grid, threads, kExtraLds, s, p);
      return;
    }
  }
  if (p.qsl && p.num_reqs <= kQslRegMax) {
    launch_fused(fused_insert_conv_kernel<D, VEC, W, BT, kQslRegs, NTX, MS, NTH>,
                 grid, threads, kExtraLds, s, p);
  } else if (p.qsl) {
    launch_fused(fused_insert_conv_kernel<D, VEC, W, BT, kQslSearch, NTX, MS, NTH>,
                 grid, threads, kExtraLds, s, p);
  } else {
    launch_fused(fused_insert_conv_kernel<D, VEC, W, BT, kQslOff, NTX, MS, NTH>,
                 grid, threads, kExtraLds, s, p);
  }
}

// Conv + window gather in one launch: built for one-generation conv launches
// (16-byte lanes, four-row tiles, streaming input loads), where the
// gather's workgroups can fill the conv's latency gaps.
template <typename D, int VEC, int W, bool MS>
static void launch_gw(const FusedGatherParams& p, uint32_t grid, uint32_t threads,
                      hipStream_t s) {
  if constexpr (VEC > 1) {
    if constexpr (W > 1) {
      if (p.guess) {
        launch_fused(fused_insert_conv_kernel<D, VEC, W, 4, kQslGuess, true, MS, false, true>,
                 grid, threads, 0, s, p);
        return;
      }
    }
    if (p.qsl && p.num_reqs <= kQslRegMax) {
      launch_fused(fused_insert_conv_kernel<D, VEC, W, 4, kQslRegs, true, MS, false, true>,
                 grid, threads, 0, s, p);
    } else if (p.qsl) {
      launch_fused(fused_insert_conv_kernel<D, VEC, W, 4, kQslSearch, true, MS, false, true>,
                 grid, threads, 0, s, p);
    } else {
      launch_fused(fused_insert_conv_kernel<D, VEC, W, 4, kQslOff, true, MS, false, true>,
                 grid, threads, 0, s, p);
    }
  }
}

template <typename D, int VEC>
static void launch_gw_w(int W, const FusedGatherParams& p, uint32_t g, uint32_t th,
                        hipStream_t s) {
  const bool ms = p.num_streams > 1;
  switch (W) {
    case 1: ms ? launch_gw<D, VEC, 1, true>(p, g, th, s) : launch_gw<D, VEC, 1, false>(p, g, th, s); break;
    case 2: ms ? launch_gw<D, VEC, 2, true>(p, g, th, s) : launch_gw<D, VEC, 2, false>(p, g, th, s); break;
    case 3: ms ? launch_gw<D, VEC, 3, true>(p, g, th, s) : launch_gw<D, VEC, 3, false>(p, g, th, s); break;
    default: ms ? launch_gw<D, VEC, 4, true>(p, g, th, s) : launch_gw<D, VEC, 4, false>(p, g, th, s); break;
  }
}

template <typename D, int VEC, int W, int BT, bool MS>
static void launch_n(const FusedParams& p, uint32_t grid, uint32_t threads, hipStream_t s) {
  // Streaming history loads are built for one-row tiles (decode).
  if constexpr (BT == 1 && W > 1) {
    if (p.nt_hist) {
      launch_q<D, VEC, W, BT, false, MS, true>(p, grid, threads, s);
      return;
    }
  }
  // Streaming input loads are built only for the 16-byte-lane 4-row tiles,
  // the shape of launches large enough to fill the chip once.
  if constexpr (VEC > 1 && BT == 4) {
    if (p.nt_x) {
      launch_q<D, VEC, W, BT, true, MS>(p, grid, threads, s);
      return;
    }
  }
  launch_q<D, VEC, W, BT, false, MS>(p, grid, threads, s);
}

template <typename D, int VEC, int W, int BT>
static void launch(const FusedParams& p, uint32_t grid, uint32_t threads, hipStream_t s) {
  if (p.num_streams > 1) launch_n<D, VEC, W, BT, true>(p, grid, threads, s);
  else launch_n<D, VEC, W, BT, false>(p, grid, threads, s);
}

template <typename D, int VEC, int W>
static void launch_bt(int bt, const FusedParams& p, uint32_t g, uint32_t th, hipStream_t s) {
  switch (bt) {
#if SCONV_FUSED_BT_MAX >= 16
    case 16: launch<D, VEC, W, 16>(p, g, th, s); break;
#endif
#if SCONV_FUSED_BT_MAX >= 8
    case 8: launch<D, VEC, W, 8>(p, g, th, s); break;
#endif
    case 4: launch<D, VEC, W, 4>(p, g, th, s); break;
    default: launch<D, VEC, W, 1>(p, g, th, s); break;
  }
}

template <typename D, int VEC>
static void launch_w(int W, int bt, const FusedParams& p, uint32_t g, uint32_t th, hipStream_t s) {
  switch (W) {
    case 1: launch_bt<D, VEC, 1>(bt, p, g, th, s); break;
    case 2: launch_bt<D, VEC, 2>(bt, p, g, th, s); break;
    case 3: launch_bt<D, VEC, 3>(bt, p, g, th, s); break;
    default: launch_bt<D, VEC, 4>(bt, p, g, th, s); break;
  }
}

// Rows per wave: the largest tile (up to SCONV_FUSED_BT_MAX) that still
// yields enough waves to keep every SIMD of the 256 CUs busy several times
// over; small batches fall back to one row per wave for parallelism.
static int pick_bt(int64_t T, int64_t slabs) {
  const int64_t kEnough = SCONV_FUSED_ENOUGH_WAVES;
  if (SCONV_FUSED_BT_MAX >= 16 && cdiv(T, 16) * slabs >= kEnough) return 16;
  if (SCONV_FUSED_BT_MAX >= 8 && cdiv(T, 8) * slabs >= kEnough) return 8;
  if (SCONV_FUSED_BT_MAX >= 4 && cdiv(T, 4) * slabs >= kEnough) return 4;
  return 1;
}

}  // namespace sconv

namespace sconv {

// Parameters of the branch-free division by d used by div_magic:
// q = (t + ((v - t) >> s1)) >> s2 with t = mulhi(v, magic) (Granlund &
// Montgomery, round-up variant; exact for every uint32 v).  d = 1: (0, 0,
// 0); d = 2^k: (1, 1, k-1); otherwise the magic number.
static void magic_for(uint32_t d, uint32_t& magic, uint32_t& s1, uint32_t& s2) {
  if (d == 1) {
    magic = 0; s1 = 0; s2 = 0;
  } else if ((d & (d - 1)) == 0) {
    magic = 1; s1 = 1; s2 = (uint32_t)__builtin_ctz(d) - 1;
  } else {
    const uint32_t l = 32 - __builtin_clz(d - 1);  // ceil(log2 d)
    magic = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
    s1 = 1;
    s2 = l - 1;
  }
}

// Shared launcher of both entry points: per-row metadata (seq_idx,
// query_start) or request offsets (qsl, num_reqs) searched in the kernel.
// With `plan` non-NULL the launch is only planned: the arguments are
// checked as for a launch, the plan is filled in and nothing is enqueued.
static int fused_launch(
    const char* fn, const sconv_stream_t* streams, int32_t num_streams, void* cache,
    int64_t num_blocks, int32_t H, int32_t N, int32_t D, int64_t cs0, int64_t cs1, int64_t cs2,
    const int64_t* positions, const int32_t* block_table, int64_t bt_row_stride,
    int32_t max_blocks, const int32_t* seq_idx, const int32_t* query_start, const int32_t* qsl,
    int32_t num_reqs, const int64_t* slot_mapping, int64_t T, int32_t W, int32_t dtype,
    hipStream_t stream, sconv_fused_plan_t* plan = nullptr,
    const sconv_window_gather_t* gather = nullptr) {
  if (T < 0) return fail(SCONV_ERR_INVALID, "%s: T < 0", fn);
  if (!valid_dtype(dtype)) return fail(SCONV_ERR_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (W < 1 || W > 4) return fail(SCONV_ERR_INVALID, "%s: W=%d outside [1, 4]", fn, W);
  if (num_streams < 1 || num_streams > kMaxStreams || !streams)
    return fail(SCONV_ERR_INVALID, "%s: num_streams=%d outside [1, %d]", fn, num_streams,
                kMaxStreams);
  if (H < 1 || N < 1 || D < 1 || num_blocks < 1 || max_blocks < 1)
    return fail(SCONV_ERR_INVALID, "%s: H, N, D, num_blocks and max_blocks must be >= 1", fn);
  if ((int64_t)num_blocks * N > INT32_MAX || (int64_t)max_blocks * N > INT32_MAX)
    return fail(SCONV_ERR_UNSUPPORTED, "%s: more than 2^31 cache slots or positions", fn);
  if (T > INT32_MAX) return fail(SCONV_ERR_UNSUPPORTED, "%s: T above 2^31", fn);
  if (cs2 < D || cs1 < 1 || cs0 < 1 || bt_row_stride < max_blocks)
    return fail(SCONV_ERR_INVALID, "%s: cache / block-table strides too small", fn);
  const int64_t es = elem_size(dtype);
  const int vec16 = (int)(16 / es);
  bool vec = cs0 % vec16 == 0 && cs1 % vec16 == 0 && cs2 % vec16 == 0 && aligned16(cache);
  int64_t C[kMaxStreams];
  for (int s = 0; s < num_streams; ++s) {
    const sconv_stream_t& q = streams[s];
    if (!valid_act(q.activation))
      return fail(SCONV_ERR_INVALID, "%s: stream %d: unknown activation %d", fn, s, q.activation);
    if (q.ws < 1) return fail(SCONV_ERR_INVALID, "%s: stream %d: ws must be >= 1", fn, s);
    if (q.off_s < 0 || (int64_t)q.off_s + q.ws > D)
      return fail(SCONV_ERR_INVALID, "%s: stream %d: range [%d, %d) outside D=%d", fn, s,
                  q.off_s, q.off_s + q.ws, D);
    for (int r = 0; r < s; ++r)
      if (q.off_s < streams[r].off_s + streams[r].ws && streams[r].off_s < q.off_s + q.ws)
        return fail(SCONV_ERR_INVALID, "%s: streams %d and %d share cache columns", fn, r, s);
    C[s] = (int64_t)H * q.ws;
    if (C[s] > INT32_MAX / 2) return fail(SCONV_ERR_UNSUPPORTED, "%s: C too large", fn);
    if (q.x_row_stride < C[s] || q.out_row_stride < C[s])
      return fail(SCONV_ERR_INVALID, "%s: stream %d: row strides must be >= C=%lld", fn, s,
                  (long long)C[s]);
    if (q.w_stride_c < 1 || q.w_stride_k < 1)
      return fail(SCONV_ERR_INVALID, "%s: stream %d: weight strides too small", fn, s);
    const bool w_packed = q.w_stride_c == W && q.w_stride_k == 1 && aligned16(q.weight);
    vec = vec && w_packed && C[s] % vec16 == 0 && q.ws % vec16 == 0 && q.off_s % vec16 == 0 &&
          q.x_row_stride % vec16 == 0 && q.out_row_stride % vec16 == 0 && aligned16(q.x) &&
          aligned16(q.out);
  }
  // The window gather, when one comes with the call: its own checks, and
  // none of its bytes may meet what the conv writes (out, cache), nor may
  // its output meet what the conv reads.
  GatherParams gp = {};
  int gvec = 1;
  bool g_empty = true;
  const int64_t es_ = elem_size(dtype);
  if (gather) {
    const sconv_window_gather_t& g = *gather;
    const int rc = gather_window_setup(fn, g.src, g.seq_len, g.conv_dim, g.src_stride_s,
                                       g.src_stride_c, g.abs_positions, g.real_count,
                                       g.max_count, g.out, g.out_slot_stride, g.d_conv, dtype, 0,
                                       &gp, &gvec, &g_empty);
    if (rc != SCONV_OK) return rc;
    if (!g_empty) {
      const int64_t gs_bytes =
          ((g.seq_len - 1) * g.src_stride_s + (int64_t)(g.conv_dim - 1) * g.src_stride_c + 1) * es_;
      const int64_t go_bytes =
          ((int64_t)(g.max_count - 1) * g.out_slot_stride + (int64_t)g.conv_dim * g.d_conv) * es_;
      const int64_t c_bytes_ = ((num_blocks - 1) * cs0 + (H - 1) * cs1 + (N - 1) * cs2 + D) * es_;
      bool bad = overlap(g.out, go_bytes, g.src, gs_bytes) ||
                 (T > 0 && (overlap(g.out, go_bytes, cache, c_bytes_) ||
                            overlap(g.src, gs_bytes, cache, c_bytes_)));
      for (int s = 0; s < num_streams && T > 0; ++s) {
        const int64_t x_bytes = ((T - 1) * streams[s].x_row_stride + C[s]) * es_;
        const int64_t o_bytes = ((T - 1) * streams[s].out_row_stride + C[s]) * es_;
        const int64_t w_bytes =
            ((C[s] - 1) * streams[s].w_stride_c + (int64_t)(W - 1) * streams[s].w_stride_k + 1) *
            es_;
        bad = bad || overlap(g.out, go_bytes, streams[s].x, x_bytes) ||
              overlap(g.out, go_bytes, streams[s].out, o_bytes) ||
              overlap(g.out, go_bytes, streams[s].weight, w_bytes) ||
              overlap(g.src, gs_bytes, streams[s].out, o_bytes);
      }
      // ... nor the conv's per-row metadata
      if (T > 0)
        bad = bad || overlap(g.out, go_bytes, positions, T * 8) ||
              overlap(g.out, go_bytes, slot_mapping, T * 8) ||
              overlap(g.out, go_bytes, seq_idx, seq_idx ? T * 4 : 0) ||
              overlap(g.out, go_bytes, query_start, query_start ? T * 4 : 0) ||
              overlap(g.out, go_bytes, qsl, qsl ? ((int64_t)num_reqs + 1) * 4 : 0);
      if (bad)
        return fail(SCONV_ERR_INVALID,
                    "%s: the gather's output overlaps its source or the conv's buffers, or "
                    "its source overlaps what the conv writes", fn);
    }
  }
  if (T == 0) {
    if (plan) {
      *plan = sconv_fused_plan_t{};
      plan->gather_mode = g_empty ? 0 : 2;
      return SCONV_OK;
    }
    if (!g_empty) {
      gather_window_launch(gp, gvec, gather->d_conv, dtype, stream);
      return check_launch(fn);
    }
    return SCONV_OK;
  }
  if (!cache || !positions || !block_table || !slot_mapping ||
      (qsl ? false : (!seq_idx || !query_start)))
    return fail(SCONV_ERR_INVALID, "%s: NULL pointer", fn);
  if (qsl && num_reqs < 1)
    return fail(SCONV_ERR_INVALID, "%s: num_reqs < 1 with %lld rows", fn, (long long)T);
  const int64_t c_bytes = ((num_blocks - 1) * cs0 + (H - 1) * cs1 + (N - 1) * cs2 + D) * es;
  for (int s = 0; s < num_streams; ++s) {
    const sconv_stream_t& q = streams[s];
    if (!q.x || !q.weight || !q.out) return fail(SCONV_ERR_INVALID, "%s: NULL pointer", fn);
    const int64_t o_bytes = ((T - 1) * q.out_row_stride + C[s]) * es;
    if (overlap(q.out, o_bytes, cache, c_bytes))
      return fail(SCONV_ERR_INVALID, "%s: out overlaps x or the cache", fn);
    for (int r = 0; r < num_streams; ++r) {
      const int64_t x_bytes = ((T - 1) * streams[r].x_row_stride + C[r]) * es;
      if (overlap(q.out, o_bytes, streams[r].x, x_bytes))
        return fail(SCONV_ERR_INVALID, "%s: out overlaps x or the cache", fn);
      if (r != s) {
        const int64_t o2 = ((T - 1) * streams[r].out_row_stride + C[r]) * es;
        if (overlap(q.out, o_bytes, streams[r].out, o2))
          return fail(SCONV_ERR_INVALID, "%s: outputs of streams %d and %d overlap", fn, r, s);
      }
    }
  }
  int VEC = vec ? vec16 : 1;
  bool narrow = false;
#if SCONV_FUSED_DECODE_LANE_BYTES == 8
  // Narrow lanes (8 bytes) for bf16 one-row tiles with W = 2 or 4: twice
  // the waves, half the arithmetic per lane after the history arrives
  // (measured slower).
  if (VEC == 8 && dtype == SCONV_BF16 && (W == 2 || W == 4) && !gather) {
    int64_t s8 = 0;
    for (int s = 0; s < num_streams; ++s) s8 += cdiv(C[s], 64 * 8);
    narrow = pick_bt(T, s8) == 1;
    if (narrow) VEC = 4;
  }
#endif

  FusedParams p = {};
  p.cache = cache; p.positions = positions; p.bt = block_table;
  p.seq_idx = seq_idx; p.slot = slot_mapping; p.qs = query_start;
  p.qsl = qsl;
  p.num_reqs = qsl ? num_reqs : 0;
  p.cs0 = cs0; p.cs1 = cs1; p.cs2 = cs2; p.bt_rs = bt_row_stride;
  p.T = T;
  p.N = N;
  magic_for(N, p.n_magic, p.n_s1, p.n_s2);
  p.num_streams = num_streams;
  int64_t slabs = 0;
  for (int s = 0; s < num_streams; ++s) {
    const sconv_stream_t& q = streams[s];
    FusedStream& f = p.st[s];
    f.x = q.x; f.w = q.weight; f.out = q.out;
    f.x_rs = q.x_row_stride; f.out_rs = q.out_row_stride;
    f.w_sc = q.w_stride_c; f.w_sk = q.w_stride_k;
    f.C = (int32_t)C[s]; f.ws = q.ws; f.off_s = q.off_s;
    f.silu = q.activation == SCONV_ACT_SILU;
    f.residual = q.use_residual != 0;
    f.slab0 = (int32_t)slabs;
    slabs += cdiv(C[s], 64 * VEC);
  }
  p.num_slabs = (int32_t)slabs;
  const int bt = narrow ? 1 : pick_bt(T, p.num_slabs);
  if (num_streams > 1 && wave_order(true, bt) == kOrderStreamInner) {
    for (int s = 1; s < num_streams; ++s)
      if (p.st[s].slab0 - p.st[s - 1].slab0 != p.st[1].slab0)
        return fail(SCONV_ERR_UNSUPPORTED, "%s: this build needs streams of equal width", fn);
    if (slabs != (int64_t)p.st[1].slab0 * num_streams)
      return fail(SCONV_ERR_UNSUPPORTED, "%s: this build needs streams of equal width", fn);
  }
  p.num_tiles = cdiv(T, bt);
  // Decode-shaped launches, where every request has the same small number
  // k of rows (k = 1 when there are no more rows than requests), guess row
  // t's request as t / k.  Larger k are prefill shapes: a coincidental
  // multiple would send most rows to the device-memory search.
  // (Only the folded forms have request offsets; they were checked above
  // to have num_reqs >= 1.)
  const bool folded = qsl != nullptr && num_reqs >= 1;
  const int64_t k = !folded || T <= num_reqs ? 1 : T / num_reqs;
  p.guess = SCONV_FUSED_BT_ROW && folded && W > 1 && k <= kGuessMaxRows &&
            (T <= num_reqs || T % num_reqs == 0) && bt_row_stride <= INT32_MAX;
  magic_for((uint32_t)(k > 0 ? k : 1), p.k_magic, p.k_s1, p.k_s2);
  // Guessed one-row tiles read block-table row t ahead (the kernel's
  // kRowAhead form): with one row per request all of it that fits in the
  // lanes' registers; otherwise (k > 1, where row t is rarely the row's
  // request) its first entry only, so that every entry the kernel reads
  // lies inside the row.  Every other form reads no row ahead.
  if (p.guess && bt == 1)
    p.bt_pref = k == 1 ? (max_blocks < kBtRowMax ? max_blocks : kBtRowMax) : 1;
  else
    p.bt_pref = 0;

  int64_t waves = p.num_tiles * p.num_slabs;
  if (waves > INT32_MAX) return fail(SCONV_ERR_UNSUPPORTED, "%s: grid too large", fn);
  // Input rows are read once, except the last W-1 rows of a tile, which the
  // next tile of the same slab reads again as its halo.  When all waves are
  // resident at once the launch is latency-bound and streaming loads win;
  // over several generations the halo re-reads must find the rows in L2.
  p.nt_x = waves <= SCONV_FUSED_NT_LOADS_MAX_WAVES;
  bool stride = false;
#if SCONV_FUSED_STRIDE
  // SCONV_FUSED_STRIDE builds: the multi-generation one-stream prefill shape
  // in striding waves, about SCONV_FUSED_STRIDE_WAVES of them.
  stride = !qsl && num_streams == 1 && VEC > 1 && bt == 4 && !p.nt_x &&
           waves > SCONV_FUSED_STRIDE_WAVES && !gather;
  if (stride) {
    p.walk_per_slab = (int32_t)((int64_t)SCONV_FUSED_STRIDE_WAVES / slabs > 0
                                    ? (int64_t)SCONV_FUSED_STRIDE_WAVES / slabs : 1);
    waves = (int64_t)p.walk_per_slab * slabs;
  }
#endif
#if SCONV_FUSED_BAND_ORDER
  // band order, exactly where the kernel takes it (multi-row tiles without
  // streaming input loads, one stream): 8 bands of ceil(tiles / 8) tiles
  if (bt > 1 && !(VEC > 1 && bt == 4 && p.nt_x) && num_streams == 1 && !stride)
    waves = 8 * cdiv(p.num_tiles, 8) * slabs;
#endif
  const uint32_t threads = waves >= 4096 || stride ? SCONV_FUSED_WG_THREADS
                                                  : SCONV_FUSED_SMALL_WG_THREADS;
  const int64_t grid = cdiv(waves, threads / 64);
  if (grid > INT32_MAX) return fail(SCONV_ERR_UNSUPPORTED, "%s: grid too large", fn);
  p.num_groups = (uint32_t)grid;
  // A history piece of one head is ws elements of a cache row.  In one-row
  // tiles (decode) whose pieces are less than a 128-byte line, streaming
  // loads measured faster: one stream 4.48 -> 4.18 us at 256 requests and
  // 19.8 -> 18.1 us at 4096; four streams of ws = 32, whose pieces share
  // lines and whose launch runs tile-major, 5.93 -> 5.53 us.  Four-row
  // tiles with whole-line pieces (spec decode) were 7-10% slower with them,
  // and so was the four-stream launch in slab-major order.
  int64_t widest = 0;  // the largest piece of any stream, in elements
  for (int s = 0; s < num_streams; ++s) widest = streams[s].ws > widest ? streams[s].ws : widest;
  p.nt_hist = SCONV_FUSED_NT_HIST && bt == 1 && widest * es < 128;
  // A one-stream decode launch whose waves are all resident at once issues
  // each row's cache insert right behind its history loads (4.150 -> 4.125
  // us at 256 requests).  Larger launches keep the stores after the
  // arithmetic: their early stores slow the history loads they travel with.
  p.early_insert = SCONV_FUSED_EARLY_INSERT == 2 ||
                   (SCONV_FUSED_EARLY_INSERT == 1 && p.nt_hist && num_streams == 1 &&
                    waves <= SCONV_FUSED_NT_LOADS_MAX_WAVES);
  p.waves_per_group = (int32_t)(threads / 64);

  // The gather runs in the conv's launch when this configuration has a
  // combined kernel: a one-generation conv in four-row tiles with 16-byte
  // lanes, and a gather on 16-byte lanes too; otherwise it is launched
  // right after the conv, on the same stream.
  const bool combined = !g_empty && VEC > 1 && bt == 4 && p.nt_x && gvec == VEC;
  if (combined) {
    gp.threads = (int32_t)threads;
    gp.cblocks = (int32_t)cdiv(gp.conv_dim, (int64_t)threads * VEC);
  }
  // One gather workgroup per (slot, channel block) item.
  const int64_t g_groups = combined ? (int64_t)gp.cblocks * gp.max_count : 0;
  if (grid + g_groups > INT32_MAX)
    return fail(SCONV_ERR_UNSUPPORTED, "%s: grid too large", fn);

  if (plan) {
    plan->gather_mode = g_empty ? 0 : combined ? 1 : 2;
    plan->lane_elems = VEC;
    plan->rows_per_tile = bt;
    plan->request_mode = p.guess ? kQslGuess
                         : !qsl ? kQslOff
                         : num_reqs <= kQslRegMax ? kQslRegs : kQslSearch;
    plan->rows_per_request = (int32_t)(k > 0 ? k : 1);
    plan->bt_row_entries = p.bt_pref;
    plan->stream_x_loads = p.nt_x;
    plan->stream_hist_loads = p.nt_hist;
    plan->early_inserts = p.early_insert;
    plan->tile_major = !slab_major_order(num_streams > 1, bt);
    plan->wg_threads = (int32_t)threads;
    plan->waves = waves;
    plan->workgroups = grid + g_groups;
    return SCONV_OK;
  }

  if (combined) {
    FusedGatherParams q;
    static_cast<FusedParams&>(q) = p;
    q.g = gp;
    q.g_dc = gather->d_conv;
    q.g_groups = (uint32_t)g_groups;
    const uint32_t all = (uint32_t)(grid + g_groups);
    q.g_interleave = SCONV_FUSED_GATHER_INTERLEAVE && grid % 8 == 0 && g_groups % 8 == 0;
    q.g_units = (uint32_t)(g_groups / 8);
    q.all_units = all / 8;
    if (dtype == SCONV_BF16) launch_gw_w<Bf16, 8>(W, q, all, threads, stream);
    else launch_gw_w<F32, 4>(W, q, all, threads, stream);
    return check_launch(fn);
  }

#if SCONV_FUSED_STRIDE
  if (stride) {
    if (dtype == SCONV_BF16) launch_stride<Bf16, 8>(W, p, (uint32_t)grid, threads, stream);
    else launch_stride<F32, 4>(W, p, (uint32_t)grid, threads, stream);
    return check_launch(fn);
  }
#endif
  if (dtype == SCONV_BF16) {
    if (VEC == 8) launch_w<Bf16, 8>(W, bt, p, (uint32_t)grid, threads, stream);
#if SCONV_FUSED_DECODE_LANE_BYTES == 8
    else if (narrow && W == 4) launch<Bf16, 4, 4, 1>(p, (uint32_t)grid, threads, stream);
    else if (narrow) launch<Bf16, 4, 2, 1>(p, (uint32_t)grid, threads, stream);
#endif
    else launch_w<Bf16, 1>(W, bt, p, (uint32_t)grid, threads, stream);
  } else {
    if (VEC == 4) launch_w<F32, 4>(W, bt, p, (uint32_t)grid, threads, stream);
    else launch_w<F32, 1>(W, bt, p, (uint32_t)grid, threads, stream);
  }
  if (!g_empty) {
    const int rc = check_launch(fn);
    if (rc != SCONV_OK) return rc;
    gather_window_launch(gp, gvec, gather->d_conv, dtype, stream);
  }
  return check_launch(fn);
}

}  // namespace sconv

static sconv_stream_t one_stream(const void* x, int64_t x_row_stride, const void* weight,
                                 int64_t w_stride_c, int64_t w_stride_k, void* out,
                                 int64_t out_row_stride, int32_t off_s, int32_t ws,
                                 int32_t activation, int32_t use_residual) {
  sconv_stream_t q;
  q.x = x; q.x_row_stride = x_row_stride; q.weight = weight;
  q.w_stride_c = w_stride_c; q.w_stride_k = w_stride_k;
  q.out = out; q.out_row_stride = out_row_stride;
  q.off_s = off_s; q.ws = ws; q.activation = activation; q.use_residual = use_residual;
  return q;
}

extern "C" int sconv_fused_insert_conv(
    const void* x, int64_t x_row_stride, const void* weight, int64_t w_stride_c,
    int64_t w_stride_k, void* cache, int64_t num_blocks, int32_t H, int32_t N, int32_t D,
    int64_t cs0, int64_t cs1, int64_t cs2, const int64_t* positions,
    const int32_t* block_table, int64_t bt_row_stride, int32_t max_blocks,
    const int32_t* seq_idx, const int64_t* slot_mapping, const int32_t* query_start, void* out,
    int64_t out_row_stride, int64_t T, int32_t off_s, int32_t ws, int32_t W, int32_t dtype,
    int32_t activation, int32_t use_residual, hipStream_t stream) {
  sconv::clear_error();
  const sconv_stream_t q = one_stream(x, x_row_stride, weight, w_stride_c, w_stride_k, out,
                                      out_row_stride, off_s, ws, activation, use_residual);
  return sconv::fused_launch("sconv_fused_insert_conv", &q, 1, cache, num_blocks, H, N, D, cs0,
                             cs1, cs2, positions, block_table, bt_row_stride, max_blocks,
                             seq_idx, query_start, nullptr, 0, slot_mapping, T, W, dtype,
                             stream);
}

extern "C" int sconv_fused_insert_conv_qsl(
    const void* x, int64_t x_row_stride, const void* weight, int64_t w_stride_c,
    int64_t w_stride_k, void* cache, int64_t num_blocks, int32_t H, int32_t N, int32_t D,
    int64_t cs0, int64_t cs1, int64_t cs2, const int64_t* positions,
    const int32_t* block_table, int64_t bt_row_stride, int32_t max_blocks,
    const int32_t* query_start_loc, int32_t num_reqs, const int64_t* slot_mapping, void* out,
    int64_t out_row_stride, int64_t T, int32_t off_s, int32_t ws, int32_t W, int32_t dtype,
    int32_t activation, int32_t use_residual, hipStream_t stream) {
  sconv::clear_error();
  if (T > 0 && !query_start_loc)
    return sconv::fail(SCONV_ERR_INVALID, "sconv_fused_insert_conv_qsl: NULL query_start_loc");
  const sconv_stream_t q = one_stream(x, x_row_stride, weight, w_stride_c, w_stride_k, out,
                                      out_row_stride, off_s, ws, activation, use_residual);
  return sconv::fused_launch("sconv_fused_insert_conv_qsl", &q, 1, cache, num_blocks, H, N, D,
                             cs0, cs1, cs2, positions, block_table, bt_row_stride, max_blocks,
                             nullptr, nullptr, query_start_loc, num_reqs, slot_mapping, T, W,
                             dtype, stream);
}

extern "C" int sconv_fused_insert_conv_streams(
    const sconv_stream_t* streams, int32_t num_streams, void* cache, int64_t num_blocks,
    int32_t H, int32_t N, int32_t D, int64_t cs0, int64_t cs1, int64_t cs2,
    const int64_t* positions, const int32_t* block_table, int64_t bt_row_stride,
    int32_t max_blocks, const int32_t* seq_idx, const int32_t* query_start,
    const int32_t* query_start_loc, int32_t num_reqs, const int64_t* slot_mapping, int64_t T,
    int32_t W, int32_t dtype, hipStream_t stream) {
  const char* fn = "sconv_fused_insert_conv_streams";
  sconv::clear_error();
  const bool per_row = seq_idx || query_start;
  if (per_row == (query_start_loc != nullptr))
    return sconv::fail(SCONV_ERR_INVALID,
                       "%s: give either seq_idx and query_start, or query_start_loc", fn);
  return sconv::fused_launch(fn, streams, num_streams, cache, num_blocks, H, N, D, cs0, cs1,
                             cs2, positions, block_table, bt_row_stride, max_blocks, seq_idx,
                             query_start, query_start_loc, num_reqs, slot_mapping, T, W, dtype,
                             stream);
}

extern "C" int sconv_fused_insert_conv_gather(
    const sconv_stream_t* streams, int32_t num_streams, void* cache, int64_t num_blocks,
    int32_t H, int32_t N, int32_t D, int64_t cs0, int64_t cs1, int64_t cs2,
    const int64_t* positions, const int32_t* block_table, int64_t bt_row_stride,
    int32_t max_blocks, const int32_t* seq_idx, const int32_t* query_start,
    const int32_t* query_start_loc, int32_t num_reqs, const int64_t* slot_mapping, int64_t T,
    int32_t W, int32_t dtype, const sconv_window_gather_t* gather, hipStream_t stream) {
  const char* fn = "sconv_fused_insert_conv_gather";
  sconv::clear_error();
  if (!gather) return sconv::fail(SCONV_ERR_INVALID, "%s: NULL gather", fn);
  const bool per_row = seq_idx || query_start;
  if (per_row == (query_start_loc != nullptr))
    return sconv::fail(SCONV_ERR_INVALID,
                       "%s: give either seq_idx and query_start, or query_start_loc", fn);
  return sconv::fused_launch(fn, streams, num_streams, cache, num_blocks, H, N, D, cs0, cs1,
                             cs2, positions, block_table, bt_row_stride, max_blocks, seq_idx,
                             query_start, query_start_loc, num_reqs, slot_mapping, T, W, dtype,
                             stream, nullptr, gather);
}

extern "C" int sconv_fused_plan(
    const sconv_stream_t* streams, int32_t num_streams, void* cache, int64_t num_blocks,
    int32_t H, int32_t N, int32_t D, int64_t cs0, int64_t cs1, int64_t cs2,
    const int64_t* positions, const int32_t* block_table, int64_t bt_row_stride,
    int32_t max_blocks, const int32_t* seq_idx, const int32_t* query_start,
    const int32_t* query_start_loc, int32_t num_reqs, const int64_t* slot_mapping, int64_t T,
    int32_t W, int32_t dtype, const sconv_window_gather_t* gather, sconv_fused_plan_t* plan) {
  const char* fn = "sconv_fused_plan";
  sconv::clear_error();
  if (!plan) return sconv::fail(SCONV_ERR_INVALID, "%s: NULL plan", fn);
  const bool per_row = seq_idx || query_start;
  if (per_row == (query_start_loc != nullptr))
    return sconv::fail(SCONV_ERR_INVALID,
                       "%s: give either seq_idx and query_start, or query_start_loc", fn);
  return sconv::fused_launch(fn, streams, num_streams, cache, num_blocks, H, N, D, cs0, cs1,
                             cs2, positions, block_table, bt_row_stride, max_blocks, seq_idx,
                             query_start, query_start_loc, num_reqs, slot_mapping, T, W, dtype,
                             nullptr, plan, gather);
}
