// Dispatch schedule (MoK paper "Mixture-of-Kittens: MoE Megakernel for
// NVL72s", §3.1 "Scheduling", Algorithm 1) and the per-minibatch GEMM tile
// lists derived from it, on gfx950.
//
// Algorithm 1 orders the local routes by expert l first, then by ordinal o
// (how many routes from rank r to expert l precede this one), then by source
// rank r; its closed form places route (r, j) at
//   S_l + sum_{r'} min(M[r'][l], o) + #{r' < r : M[r'][l] > o}.
// Three kernels build it without order-dependent atomics:
//   count : per chunk of a source rank's routes, the chunk-local ordinal of
//           every local route (wave ballots + per-wave counts in LDS, taken in
//           wave order) and the chunk's per-expert histogram;
//   scan  : per (r, l) exclusive prefix over chunks -> chunk bases and M[r][l]
//           (a few threads per pair, each over a run of chunks); counts and
//           expert offsets S_l (block-wide scan);
//   place : o = chunk base + local ordinal, then the closed form above (M
//           staged in LDS); writes the table row and its inverse.

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

constexpr int kSchedChunk = 1024;  // routes per count block
constexpr int kMaxExperts = 1024;

// Exclusive scan of one int per thread over a block of 1024 threads.
__device__ int block_exclusive_scan_1024(int v, int* total) {
  __shared__ int wave_sum[16];
  const int lane = lane_id(), w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) wave_sum[w] = x;
  __syncthreads();
  if (w == 0) {
    int s = lane < 16 ? wave_sum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (lane < 16) wave_sum[lane] = s;  // inclusive prefix of wave totals
  }
  __syncthreads();
  const int before = (w > 0 ? wave_sum[w - 1] : 0) + x - v;
  if (total) *total = wave_sum[15];
  __syncthreads();
  return before;
}

__global__ __launch_bounds__(256) void sched_count_kernel(const int32_t* __restrict__ A, int NK, int c, int L,
                                                          int E_total, int nch, int32_t* __restrict__ ord_local,
                                                          int32_t* __restrict__ chunk_cnt, int* err) {
  __shared__ int run[kMaxExperts];
  __shared__ int wcnt[4][kMaxExperts];
  const int r = blockIdx.y, ch = blockIdx.x;
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  for (int i = tid; i < L; i += 256) {
    run[i] = 0;
    wcnt[0][i] = wcnt[1][i] = wcnt[2][i] = wcnt[3][i] = 0;
  }
  __syncthreads();
  const int nbits = 32 - __clz(L);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int sub = 0; sub < kSchedChunk / 256; ++sub) {
    const int j = ch * kSchedChunk + sub * 256 + tid;
    int l = -1;
    if (j < NK) {
      const int a = A[static_cast<int64_t>(r) * NK + j];
      if (a < 0 || a >= E_total)
        raise_error(err, kErrExpertRange);
      else if (a >= c * L && a < c * L + L)
        l = a - c * L;
    }
    // lanes of this wave routed to the same local expert
    uint64_t same = __ballot(l >= 0);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (l >> bit) & 1;
      const uint64_t bal = __ballot(set);
      same &= set ? bal : ~bal;
    }
    const int rank = __popcll(same & lt_mask);
    if (l >= 0 && rank == 0) wcnt[w][l] = __popcll(same);
    __syncthreads();
    if (l >= 0) {
      int o = run[l] + rank;
      for (int w2 = 0; w2 < w; ++w2) o += wcnt[w2][l];
      ord_local[static_cast<int64_t>(r) * NK + j] = o;
    }
    __syncthreads();
    for (int i = tid; i < L; i += 256) {
      run[i] += wcnt[0][i] + wcnt[1][i] + wcnt[2][i] + wcnt[3][i];
      wcnt[0][i] = wcnt[1][i] = wcnt[2][i] = wcnt[3][i] = 0;
    }
    __syncthreads();
  }
  for (int i = tid; i < L; i += 256) chunk_cnt[(static_cast<int64_t>(r) * nch + ch) * L + i] = run[i];
}

__global__ __launch_bounds__(1024) void sched_scan_kernel(int R, int L, int nch, int NK, int32_t* __restrict__ chunk_cnt,
                                                          int32_t* __restrict__ Mmat, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets, int64_t max_rows, int* err) {
  __shared__ int Ms[kMaxExperts];  // M[r][l] (R * L = E_total <= kMaxExperts)
  const int tid = threadIdx.x;
  // G threads (adjacent lanes) share one (r, l) pair, each taking a run of
  // chunks; the chunk counts of a run are loaded in batches of 8 so that the
  // loads are in flight together
  const int pairs = R * L;
  int G = 1;
  while (G < 16 && pairs * G * 2 <= 1024) G *= 2;
  const int pair = tid / G, g = tid % G;
  const bool active = pair < pairs && NK > 0;  // no count pass ran when there are no routes
  const int per = (nch + G - 1) / G;
  const int ch0 = g * per, ch1 = min(nch, ch0 + per);
  const int64_t row = static_cast<int64_t>(pair / (L > 0 ? L : 1)) * nch;  // first chunk entry of rank r
  const int l = pair % (L > 0 ? L : 1);
  auto at = [&](int ch) { return (row + ch) * L + l; };
  int part = 0;
  for (int ch = ch0; active && ch < ch1; ch += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ch + i < ch1 ? chunk_cnt[at(ch + i)] : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) part += v[i];
  }
  // exclusive prefix of the runs' sums over the pair's G threads
  int incl = part;
  for (int off = 1; off < G; off <<= 1) {
    const int y = __shfl_up(incl, off, G);
    if (g >= off) incl += y;
  }
  int base = incl - part;
  const int pair_total = __shfl(incl, G - 1, G);
  // chunk counts -> exclusive chunk bases, in chunk order
  for (int ch = ch0; active && ch < ch1; ch += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ch + i < ch1 ? chunk_cnt[at(ch + i)] : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (ch + i < ch1) chunk_cnt[at(ch + i)] = base;
      base += v[i];
    }
  }
  if (pair < pairs && g == 0) {
    Mmat[pair] = pair_total;
    Ms[pair] = pair_total;
  }
  __syncthreads();
  int cnt = 0;
  if (tid < L) {
    for (int r = 0; r < R; ++r) cnt += Ms[r * L + tid];
    counts[tid] = cnt;
  }
  int total = 0;
  const int start = block_exclusive_scan_1024(cnt, &total);
  if (tid < L) offsets[tid] = start;
  if (tid == 0) {
    offsets[L] = total;
    if (total > max_rows) raise_error(err, kErrRowOverflow);
  }
}

__global__ __launch_bounds__(256) void sched_place_kernel(const int32_t* __restrict__ A, int R, int NK, int c, int L,
                                                          int nch, const int32_t* __restrict__ ord_local,
                                                          const int32_t* __restrict__ chunk_base,
                                                          const int32_t* __restrict__ Mmat,
                                                          const int32_t* __restrict__ offsets, int64_t max_rows,
                                                          int32_t* __restrict__ sched_src,
                                                          int32_t* __restrict__ route_dst, int* err) {
  __shared__ int Ms[kMaxExperts];  // M[r][l] (R * L = E_total <= kMaxExperts)
  for (int i = threadIdx.x; i < R * L; i += 256) Ms[i] = Mmat[i];
  __syncthreads();
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= static_cast<int64_t>(R) * NK) return;
  const int r = static_cast<int>(gid / NK), j = static_cast<int>(gid % NK);
  const int a = A[gid];
  if (a < c * L || a >= c * L + L) {
    route_dst[gid] = -1;
    return;
  }
  const int l = a - c * L;
  const int o = chunk_base[(static_cast<int64_t>(r) * nch + j / kSchedChunk) * L + l] + ord_local[gid];
  int p = 0;
  for (int r2 = 0; r2 < R; ++r2) {
    const int m = Ms[r2 * L + l];
    p += m < o ? m : o;
    if (r2 < r && m > o) ++p;
  }
  const int64_t pos = static_cast<int64_t>(offsets[l]) + p;
  if (pos < max_rows) {
    sched_src[pos] = static_cast<int32_t>(gid);
    route_dst[gid] = static_cast<int32_t>(pos);
  } else {
    route_dst[gid] = -1;
    raise_error(err, kErrRowOverflow);
  }
}

hipError_t launch_schedule(const int32_t* routes, int R, int NK, int c, int L, int E_total, int64_t max_rows,
                           int32_t* counts, int32_t* offsets, int32_t* sched_src, int32_t* route_dst,
                           const SchedScratch& s, int* err, hipStream_t stream) {
  const int nch = sched_chunks(NK);
  if (NK > 0) {
    sched_count_kernel<<<dim3(nch, R), 256, 0, stream>>>(routes, NK, c, L, E_total, nch, s.ord_local, s.chunk_cnt,
                                                         err);
  }
  sched_scan_kernel<<<1, 1024, 0, stream>>>(R, L, nch, NK, s.chunk_cnt, s.M, counts, offsets, max_rows, err);
  const int64_t n = static_cast<int64_t>(R) * NK;
  if (n > 0) {
    sched_place_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(
        routes, R, NK, c, L, nch, s.ord_local, s.chunk_cnt, s.M, offsets, max_rows, sched_src, route_dst, err);
  }
  return hipGetLastError();
}

int sched_chunks(int NK) { return NK > 0 ? (NK + kSchedChunk - 1) / kSchedChunk : 1; }

// ----------------------------------------------------------------------------
// Tile lists: for minibatch m (positions m*b .. min(m*b+b, P)-1), every expert
// segment that overlaps it is cut into n = ceil(rows / BM) row tiles of nearly
// equal height (rounded up to 32 rows, the MFMA block), in expert order.  With
// balanced heights the tiles of one segment run at the same pace, so the
// workgroups that read the same expert weights stay together and share them in
// L2 instead of re-fetching them from HBM.  Entry = {expert | (n << 10), first
// position, rows, index of this expert's first tile}; the GEMM kernels order
// their work by it.
//
// XCD runs.  The GEMM kernels cut a list's work items (N blocks of each row
// tile) into 8 contiguous runs, one per XCD.  Equal item counts are equal work
// only while the tiles have nearly equal heights; under skewed routing a list
// holds the full tiles of a few large experts and many short tiles of small
// ones, and the XCDs that get the large experts' tiles would run longest.  So
// the runs are cut by cost: a tile of r rows is taken to cost ceil(r / 32) +
// BM / 32 units (its 32-row MFMA blocks, plus the weight slab and the tile of
// activation rows it streams whatever its height), and boundary j (j = 1 ..
// 7) is the position where the running cost reaches j / 8 of the list's
// total, placed inside its expert's tiles in proportion to cost, in
// 1/kTileRunFrac of a tile.  (Cutting only at tile-group starts measured
// slower on lists of a few large experts: too coarse with about a dozen tiles
// per XCD.)  The boundaries rise with j, so the runs partition the items;
// which XCD runs an item does not change its result.  Then each run is held
// to at most `cap` tiles (tile_run_cap), the most its XCD's workgroups cover
// in the up/gate launch: boundary j is clamped, in order, into [runs[j - 1],
// runs[j - 1] + cap] and no lower than count - (8 - j) cap, so that the runs
// after it can still hold the rest (8 cap >= count makes the range
// non-empty).  Balanced runs stay far inside the cap: a tile costs between 1
// and 2 times BM / 32 units, so a run of one eighth of the cost holds at most
// about a quarter of the tiles.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets, int L, int64_t b,
                                                           int64_t max_rows, int BM, int max_tiles,
                                                           int4* __restrict__ tiles, int32_t* __restrict__ tile_count,
                                                           int32_t* __restrict__ runs) {
  const int m = blockIdx.x, l = threadIdx.x;
  // rows past max_rows were never placed (the schedule flagged the overflow)
  const int64_t P = offsets[L] < max_rows ? offsets[L] : max_rows;
  const int64_t lo = static_cast<int64_t>(m) * b;
  const int64_t hi = lo + b < P ? lo + b : P;
  int64_t s_lo = 0, s_hi = 0;
  int n = 0;
  if (l < L) {
    s_lo = offsets[l] > lo ? offsets[l] : lo;
    s_hi = offsets[l + 1] < hi ? offsets[l + 1] : hi;
    if (s_hi > s_lo) n = static_cast<int>((s_hi - s_lo + BM - 1) / BM);
  }
  int total = 0;
  const int start = block_exclusive_scan_1024(n, &total);
  int4* out = tiles + static_cast<int64_t>(m) * max_tiles;
  if (n > 0) {
    const int64_t len = s_hi - s_lo;
    int64_t h = (len + n - 1) / n;
    h = (h + 31) / 32 * 32;  // <= BM since BM is a multiple of 32
    for (int i = 0; i < n; ++i) {
      if (start + i >= max_tiles) break;
      const int64_t p0 = s_lo + static_cast<int64_t>(i) * h;
      const int64_t rows = s_hi - p0 < h ? s_hi - p0 : h;
      if (rows <= 0) break;  // unreachable: n tiles of height h >= len / n cover the segment
      out[start + i] = make_int4(l | (n << 10), static_cast<int>(p0), static_cast<int>(rows), start);
    }
  }
  const int count = total < max_tiles ? total : max_tiles;
  if (l == 0) tile_count[m] = count;
  if (!runs) return;  // uniform: every thread of the block returns here

  // cost units of this expert's tiles: all but the last are h rows high
  int cost = 0;
  if (n > 0) {
    const int64_t len = s_hi - s_lo;
    const int64_t h = ((len + n - 1) / n + 31) / 32 * 32;
    const int last = static_cast<int>((len - (n - 1) * h + 31) / 32);
    cost = (n - 1) * static_cast<int>(h / 32 + BM / 32) + last + BM / 32;
  }
  int total_cost = 0;
  const int before = block_exclusive_scan_1024(cost, &total_cost);
  const int count_pos = count * kTileRunFrac;
  __shared__ int bound[kTileRunBounds];  // boundary j, written by the expert whose cost range holds j / 8 of it
  if (cost > 0) {
    for (int j = 1; j < kXcds; ++j) {
      const int target = static_cast<int>(static_cast<int64_t>(total_cost) * j / kXcds);
      if (target < before || target >= before + cost) continue;  // another expert's
      const int64_t into = static_cast<int64_t>(target - before) * n * kTileRunFrac;
      const int64_t pos = static_cast<int64_t>(start) * kTileRunFrac + (into + cost / 2) / cost;
      bound[j] = pos < count_pos ? static_cast<int>(pos) : count_pos;
    }
  }
  __syncthreads();
  if (l == 0) {
    const int64_t cap = static_cast<int64_t>(tile_run_cap(max_tiles)) * kTileRunFrac;
    int32_t* r = runs + static_cast<int64_t>(m) * kTileRunBounds;
    int64_t prev = 0;
    r[0] = 0;
    for (int j = 1; j < kXcds; ++j) {
      int64_t v = total_cost > 0 ? bound[j] : 0;  // no tiles: every run is empty
      const int64_t lo = count_pos - (kXcds - j) * cap;
      v = v < lo ? lo : v;
      v = v < prev ? prev : v;
      v = v > prev + cap ? prev + cap : v;
      r[j] = static_cast<int32_t>(v);  // <= count_pos
      prev = v;
    }
    r[kXcds] = count_pos;
  }
}

// Dense tile list: one segment [0, rows) of expert 0, split as the routed
// lists split an expert segment (equal heights rounded up to 32, at most BM).
__global__ void dense_tiles_kernel(int64_t rows, int BM, int4* __restrict__ tiles, int32_t* __restrict__ tile_count) {
  const int n = static_cast<int>((rows + BM - 1) / BM);
  int64_t h = (rows + n - 1) / n;
  h = (h + 31) / 32 * 32;  // <= BM since BM is a multiple of 32
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t p0 = static_cast<int64_t>(i) * h;
    const int64_t r = rows - p0 < h ? rows - p0 : h;  // > 0: (n - 1) * h < rows
    tiles[i] = make_int4(n << 10, static_cast<int>(p0), static_cast<int>(r), 0);
  }
  if (threadIdx.x == 0) *tile_count = n;
}

int dense_tiles_bound(int64_t rows, int BM) { return rows > 0 ? static_cast<int>((rows + BM - 1) / BM) : 1; }

hipError_t launch_dense_tiles(int64_t rows, int BM, int4* tiles, int32_t* tile_count, hipStream_t stream) {
  if (rows <= 0 || BM <= 0 || BM % 32 || rows >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if ((rows + BM - 1) / BM >= (1 << 21)) return hipErrorInvalidValue;  // the tile count shares a word with the expert id
  dense_tiles_kernel<<<1, 256, 0, stream>>>(rows, BM, tiles, tile_count);
  return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t* offsets, int L, int64_t b, int64_t max_rows, int BM, int n_minibatches,
                              int max_tiles, int4* tiles, int32_t* tile_count, int32_t* runs, hipStream_t stream) {
  static_assert(kTileRunBounds == kXcds + 1, "one run per XCD");
  if (n_minibatches <= 0) return hipSuccess;
  // run positions (kTileRunFrac per tile) are int32
  if (runs && static_cast<int64_t>(max_tiles) * kTileRunFrac >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  build_tiles_kernel<<<n_minibatches, 1024, 0, stream>>>(offsets, L, b, max_rows, BM, max_tiles, tiles, tile_count,
                                                         runs);
  return hipGetLastError();
}

}  // namespace moe
