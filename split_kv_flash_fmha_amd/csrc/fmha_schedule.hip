// Length-aware tile schedule for prefill ("Adds variable sequence lengths to
// the Hopper CuTe DSL FMHA example", Performance (GH200): a static
// round-robin assignment over the max-length grid balances skewed lengths
// poorly, and a length-aware schedule is named as the follow-up).
//
// One workgroup reads cu_seqlens on the device and builds a table that maps
// each position of the attention grid to a tile:
//  * the cost of a tile is the number of key blocks its key range spans (the
//    kernel's own range arithmetic: causal and window bounds of its first and
//    last row) plus one for its fixed work; a sequence's cost is the sum over
//    its query tiles;
//  * groups are (sequence, kv head): every tile of a group reads the same K
//    and V, so a group's tiles stay together on one XCD, one after the other,
//    and reuse K/V in that XCD's L2; last tile first when it costs at least
//    as much as the first (causal, right window), else first tile first (a
//    left-only window), i.e. costliest first where costs are monotone along
//    the sequence.  Ordering single tiles by cost instead scatters a
//    group's tiles over the launch: with many sequences (K/V far beyond the
//    caches) that re-fetched K/V from HBM and ran 40 % slower than the plain
//    grouped order;
//  * groups are taken longest first and dealt to the 8 XCDs in snake order
//    (0..7, 7..0, ...), a longest-processing-time-first assignment: each XCD
//    holds its 1/8 share of the cost within one group's cost (each round
//    gives it one group no larger than any of the previous round's); grid
//    position 8 j + x holds
//    item j of XCD x's list (the hardware sends block i to XCD i % 8);
//  * a list has room for positions / 8 items.  Dealing by cost does not
//    bound a list's tile count (a sequence with many query rows and few keys
//    is cheap but has many tiles), so the items of a list past its room are
//    moved, in order, to the free ends of the lists with room left (lowest
//    XCD first); the host sizes the positions so that the rooms together
//    hold every tile.  Positions past the end of a list hold no tile (-1).
// The grid thus covers only the tiles that exist (the plain grouped order
// launches batch x kv heads x the longest sequence's tiles).
//
// Table (int32, in the workspace): [0] positions, [1 + x] how far a
// persistent launch has claimed XCD x's list (set to 0 here), [16 + 2i]
// sequence of position i or -1, [17 + 2i] kv head << 20 | query tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fmha_fwd_kernel.h"
#include "fmha_params.h"

namespace fmha {

namespace {

constexpr int kSchedThreads = 1024;
constexpr int kPerXcd = kSchedThreads / kXcds;  // threads scanning one XCD's list

// cost of query tile t of a sequence (sq queries, sk > 0 keys)
__device__ __forceinline__ int tile_cost(const FwdParams& p, int sq, int sk, int t, int rows_per_tile,
                                         int key_block) {
  const int G = p.group;
  const int rows = sq * G;
  const int row0 = t * rows_per_tile;
  const int last = min(row0 + rows_per_tile, rows) - 1;
  const int shift = sk - sq;
  const int i_lo = row0 / G, i_hi = last / G;
  const int lo = p.wl >= 0 ? max(i_lo + shift - p.wl, 0) : 0;
  const int hi = p.wr >= 0 ? min(i_hi + shift + p.wr, sk - 1) : sk - 1;
  const int jb = lo / key_block * key_block;
  const int blocks = hi + 1 > jb ? (hi + 1 - jb + key_block - 1) / key_block : 0;
  return blocks + 1;
}

// positions: entries of the table (the attention grid); batch <= kSchedThreads
__global__ __launch_bounds__(kSchedThreads) void fmha_schedule_kernel(FwdParams p, int rows_per_tile, int key_block,
                                                                       int positions, int32_t* tab) {
  __shared__ long long s_cost[kSchedThreads];
  __shared__ int s_nt[kSchedThreads], s_desc[kSchedThreads], s_order[kSchedThreads];
  __shared__ int s_part[kSchedThreads / 64];
  __shared__ int s_len[kXcds], s_end[kXcds];
  const int tid = threadIdx.x;
  const int G = p.group;
  const int batch = p.batch;

  // per sequence: tiles, cost, and whether its costliest tiles are its last
  long long cost = 0;
  int nt = 0, desc = 1;
  if (tid < batch) {
    WorkItem w;
    seq_span(p, tid, w);
    nt = (w.sq > 0 && w.sk > 0) ? (w.sq * G + rows_per_tile - 1) / rows_per_tile : 0;
    for (int t = 0; t < nt; ++t) cost += tile_cost(p, w.sq, w.sk, t, rows_per_tile, key_block);
    if (nt > 1)
      desc = tile_cost(p, w.sq, w.sk, nt - 1, rows_per_tile, key_block) >=
             tile_cost(p, w.sq, w.sk, 0, rows_per_tile, key_block);
  }
  s_cost[tid] = cost;
  s_nt[tid] = nt;
  s_desc[tid] = desc;
  __syncthreads();
  // rank by cost, longest first (ties by index): s_order[rank] = sequence
  if (tid < batch) {
    int rank = 0;
    for (int j = 0; j < batch; ++j) {
      const long long cj = s_cost[j];
      rank += cj > cost || (cj == cost && j < tid);
    }
    s_order[rank] = tid;
  }
  __syncthreads();

  // group k (k = rank * Hkv + kv head) goes to XCD x in round R = k / 8:
  // k = 8 R + x (R even) or 8 R + 7 - x (R odd).  Thread l of XCD x's
  // kPerXcd threads takes rounds [l * per, (l + 1) * per).
  const int H = p.hkv;
  const int ngroups = batch * H;
  const int rounds = (ngroups + kXcds - 1) / kXcds;
  const int per = (rounds + kPerXcd - 1) / kPerXcd;
  const int x = tid / kPerXcd, l = tid % kPerXcd;
  auto group_of = [&](int R) { return kXcds * R + ((R & 1) ? kXcds - 1 - x : x); };
  int mine = 0;
  for (int R = l * per; R < min(rounds, (l + 1) * per); ++R) {
    const int k = group_of(R);
    if (k < ngroups) mine += s_nt[s_order[k / H]];
  }
  // exclusive prefix of `mine` over the kPerXcd threads of this XCD (two waves)
  const int incl = wave_scan(mine);
  if ((tid & 63) == 63) s_part[tid >> 6] = incl;
  __syncthreads();
  const int first_wave = x * (kPerXcd / 64);
  int off = incl - mine;
  for (int w = first_wave; w < (tid >> 6); ++w) off += s_part[w];
  if (l == kPerXcd - 1) s_len[x] = off + mine;
  __syncthreads();

  // room per list; the items of a list past its room go to the free
  // ends of the lists with room left, overflow item q to the q-th free slot
  // counted from XCD 0 (the rooms hold every tile: positions is sized so)
  const int room = positions / kXcds;
  int over_before = 0;  // overflow items of the lists before this one
  for (int y = 0; y < x; ++y) over_before += max(s_len[y] - room, 0);
  auto place = [&](int j) {  // position of item j of this XCD's list
    if (j < room) return kXcds * j + x;
    int q = over_before + (j - room);
    for (int y = 0; y < kXcds; ++y) {
      const int free_y = max(room - s_len[y], 0);
      if (q < free_y) return kXcds * (s_len[y] + q) + y;
      q -= free_y;
    }
    return positions;  // unreachable with the host's sizing; dropped rather than written out of range
  };
  for (int R = l * per; R < min(rounds, (l + 1) * per); ++R) {
    const int k = group_of(R);
    if (k >= ngroups) continue;
    const int b = s_order[k / H], h = k % H, n = s_nt[b];
    for (int j = 0; j < n; ++j) {
      const int pos = place(off + j);
      if (pos < positions) {
        tab[kSchedHead + 2 * pos] = b;
        tab[kSchedHead + 1 + 2 * pos] = (h << 20) | (s_desc[b] ? n - 1 - j : j);
      }
    }
    off += n;
  }
  __syncthreads();
  // positions past each list's end (its own items and the overflow placed
  // there) hold no tile
  if (tid == 0) {
    int left = 0;
    for (int y = 0; y < kXcds; ++y) left += max(s_len[y] - room, 0);
    for (int y = 0; y < kXcds; ++y) {
      const int free_y = max(room - s_len[y], 0), took = min(free_y, left);
      s_end[y] = min(s_len[y], room) + took;
      left -= took;
    }
  }
  __syncthreads();
  for (int pos = tid; pos < positions; pos += kSchedThreads)
    if (pos / kXcds >= s_end[pos % kXcds]) tab[kSchedHead + 2 * pos] = -1;
  if (tid == 0) tab[0] = positions;
  if (tid < kXcds) tab[1 + tid] = 0;
}

}  // namespace

hipError_t launch_schedule(const FwdParams& p, int rows_per_tile, int key_block, int positions, int32_t* table,
                           hipStream_t stream) {
  hipLaunchKernelGGL(fmha_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, p, rows_per_tile, key_block,
                     positions, table);
  return hipGetLastError();
}

}  // namespace fmha
