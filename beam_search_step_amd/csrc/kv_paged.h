// kv_paged.h -- part of libbeamstep.so, included once by beamstep.hip.
//
// The paged KV cache with copy on write: K6, K7.
#pragma once

namespace {

// ---------------------------------------------------------------------------
// K6/K7: paged KV cache -- block tables with copy on write
// ---------------------------------------------------------------------------

constexpr int kPagedMaxBlocks = 4096;  // blocks per item (LDS reference counts)
constexpr int kPagedMaxTable = 2048;   // W * max_blocks (LDS table copies)

struct PagedDev {
  int* table;     // [B*W][mb] global block ids, -1 = none
  int* refc;      // [B*bpi] live-row references of each block
  int* freel;     // [B][bpi] stack of free global block ids
  int* nfree;     // [B]
  int* overflow;  // [1]
  int* cpy;       // [B*W][3] copy list of the step: source block, destination block, positions
  int* ncpy;      // [2] entries of the list, by step parity
};

struct K6Args {
  PagedDev pg;
  const float* s;       // [B*W] running scores after the step
  const uint8_t* done;  // [B] after the step
  const int* plan;      // [B][kPlanStride] the step's reorder plan
  int W, bs, bpi, mb, t;
};

// One workgroup per item. The item's table, reference counts and free list
// are staged in LDS; the new table is formed from the old one and the plan,
// references are added before old ones are dropped (a block both gains and
// loses references without being freed in between), and a block whose count
// reaches zero goes back to the free list. Then wave 0 makes position t
// writable for every live slot.
__device__ __forceinline__ void paged_update_item(const K6Args& a, int b, int tid) {
  __shared__ int refc[kPagedMaxBlocks];
  __shared__ int fstack[kPagedMaxBlocks];
  __shared__ int told[kPagedMaxTable];
  __shared__ int tnew[kPagedMaxTable];
  __shared__ int par[kMaxBeam];
  __shared__ int plan_sh[2 + 2 * kMaxBeam];
  __shared__ int nfree_sh;
  const int W = a.W, mb = a.mb, bpi = a.bpi, t = a.t, bs = a.bs;
  const int base = b * bpi;          // the item's first global block id
  const int nb = (t + bs - 1) / bs;  // blocks holding positions [0, t)
  const int nt = W * mb;
  const PagedDev& pg = a.pg;
  const int* plan = a.plan + b * kPlanStride;
  const bool item_done = a.done[b] != 0;
  const int nf = min(max(pg.nfree[b], 0), bpi);
  for (int e = tid; e < bpi; e += kThreads) refc[e] = pg.refc[base + e];
  for (int e = tid; e < nf; e += kThreads) fstack[e] = pg.freel[base + e];
  for (int e = tid; e < nt; e += kThreads) {
    const int v = pg.table[(int64_t)b * nt + e];
    told[e] = (v >= base && v < base + bpi) ? v : -1;  // only the item's own blocks
  }
  if (tid < 2 + 2 * kMaxBeam) plan_sh[tid] = plan[tid];  // staged with the other loads
  if (tid == 0) nfree_sh = nf;
  __syncthreads();
  if (tid < W) {  // parent of each slot: itself unless the plan moves it
    int pp = tid;
    if (plan_sh[1] > 0)
      for (int q = 0; q < plan_sh[0]; ++q)
        if ((plan_sh[2 + kMaxBeam + q] >> tid) & 1) pp = plan_sh[2 + q];
    par[tid] = pp;
  }
  __syncthreads();

  // new table: a live slot of a running item takes its parent's blocks
  // [0, nb); rows of dead slots and of finished items hold nothing
  for (int e = tid; e < nt; e += kThreads) {
    const int i = e / mb, k = e - i * mb;
    int v = -1;
    if (!item_done && a.s[b * W + i] > -kInf && k < nb) v = told[par[i] * mb + k];
    tnew[e] = v;
  }
  __syncthreads();
  for (int e = tid; e < nt; e += kThreads)
    if (tnew[e] >= 0) atomicAdd(&refc[tnew[e] - base], 1);
  __syncthreads();
  for (int e = tid; e < nt; e += kThreads)
    if (told[e] >= 0 && atomicSub(&refc[told[e] - base], 1) == 1) {
      const int slot = atomicAdd(&nfree_sh, 1);
      if (slot < kPagedMaxBlocks) fstack[slot] = told[e];
    }
  __syncthreads();

  // position t: a fresh block at a block boundary; inside a block that a
  // lower live slot also holds, a private copy of its first t % bs positions
  if (tid < 64) {
    const int lane = tid;
    const int blk = t / bs, off = t - blk * bs;
    const bool live = lane < W && !item_done && a.s[b * W + lane] > -kInf;
    const int cur = live ? tnew[lane * mb + blk] : -1;
    bool shared = false;
    for (int j = 0; j < W; ++j) {
      const bool lj = !item_done && a.s[b * W + j] > -kInf;
      if (j < lane && lj && cur >= 0 && tnew[j * mb + blk] == cur) shared = true;
    }
    const bool alloc = live && (off == 0 || cur < 0 || shared);
    const bool copy = live && off > 0 && cur >= 0 && shared;
    const uint64_t below = (lane == 0) ? 0 : (~(uint64_t)0 >> (64 - lane));
    const uint64_t am = __ballot(alloc);
    const int rank = __popcll(am & below);
    const int avail = min(nfree_sh, bpi);
    int nbk = -1;
    if (alloc && rank < avail) nbk = fstack[avail - 1 - rank];
    if (nbk < base || nbk >= base + bpi) nbk = -1;  // only the item's own blocks
    const bool got = nbk >= 0;
    if (alloc && !got) {  // out of blocks: the slot is left without one
      pg.overflow[0] = 1;
      if (cur >= 0) {
        tnew[lane * mb + blk] = -1;
        atomicSub(&refc[cur - base], 1);  // still held by a lower slot
      }
    }
    const uint64_t cm = __ballot(copy && got);
    // the item's copies go to the step's global list (one atomic per item);
    // the other parity's count is cleared for the next step
    int cbase = 0;
    if (lane == 0 && cm) cbase = atomicAdd(&pg.ncpy[t & 1], __popcll(cm));
    cbase = __builtin_amdgcn_readfirstlane(cbase);
    if (b == 0 && lane == 0) pg.ncpy[(t + 1) & 1] = 0;
    __builtin_amdgcn_wave_barrier();
    if (got) {
      tnew[lane * mb + blk] = nbk;
      refc[nbk - base] = 1;
      if (copy) {
        atomicSub(&refc[cur - base], 1);
        int* c = pg.cpy + ((int64_t)cbase + __popcll(cm & below)) * 3;
        c[0] = cur;
        c[1] = nbk;
        c[2] = off;
      }
    }
    if (lane == 0) {
      const int used = __popcll(am) < avail ? __popcll(am) : avail;
      nfree_sh = avail - used;
    }
  }
  __syncthreads();

  for (int e = tid; e < bpi; e += kThreads) pg.refc[base + e] = refc[e];
  const int nf2 = min(nfree_sh, bpi);
  for (int e = tid; e < nf2; e += kThreads) pg.freel[base + e] = fstack[e];
  for (int e = tid; e < nt; e += kThreads) pg.table[(int64_t)b * nt + e] = tnew[e];
  if (tid == 0) pg.nfree[b] = nf2;
}

__global__ __launch_bounds__(kThreads) void k6_paged_reorder(K6Args a) {
  paged_update_item(a, blockIdx.x, threadIdx.x);
}

// K2 and K6 in one launch, for a step whose cache is paged: the workgroup of
// item b runs the selection and finalize of the step, then (after a barrier,
// which also makes the step's scores, done flag and plan, written to global
// memory by its wave 0, visible to every wave of the workgroup) the item's
// table update. It saves K6's launch (measured: 9.4 us for the two, against
// 5.6 + 5.8 us as separate launches at the Llama-3-8B shape; loading the
// item's paged state into registers before the selection, to overlap its
// round trip, made it slower, 9.9 us).
template <int WMAX, int H>
__global__ __launch_bounds__(kThreads) void k2_select_finalize_paged(K2Args a, K6Args a6) {
  select_finalize_item<WMAX, H>(a);
  __syncthreads();
  paged_update_item(a6, blockIdx.x, threadIdx.x);
}

struct K7Args {
  char* pools[kMaxPlanesPerLaunch];
  int n_planes;
  int64_t block_stride, pos_stride;
  int words_per_pos;
  int tiles;             // word tiles of a copy of block_size - 1 positions
  int groups;            // groups of kCopyPlanes pools
  const int* cpy;
  const int* ncpy;
  int parity;
  int max_copies;        // capacity of the list: B*W
};

// The copies on write of the step: a fixed grid walks the units (copy, word
// tile, group of kCopyPlanes pools) of the step's list; a thread moves one
// word of each pool of its unit's group, all loads issued before the first
// store. The grid is sized so that a workgroup rarely takes more than one
// unit, since a workgroup's next unit waits for its previous stores (with
// 256-thread workgroups, 1024 of them measured 11% faster per step than 256
// with blocks of 16 positions, 18% with blocks of 32; 2048 no faster).
// Workgroups are one wave, as in the contiguous reorder: 4096 of 64 threads
// gave 44,867-45,581 beam steps/s against 43,997-44,554 for 1024 of 256 at the
// Llama-3-8B shape (blocks of 16, three runs each), 2048 of 64 in between. Loads and stores carry the nontemporal
// hint, as the contiguous reorder's do (every word is read once and written
// once): 42,588-42,856 beam steps/s against 40,534-40,821 with plain ones at
// the Llama-3-8B shape (blocks of 16, three runs each).
constexpr int kCopyPlanes = 8;
constexpr int kCopyGrid = 4096;
constexpr int kK7Threads = 64;
template <int WORD>
__global__ __launch_bounds__(kK7Threads) void k7_paged_copy(K7Args a) {
  using WT = typename Word<WORD>::type;
  const int units = min(a.ncpy[a.parity], a.max_copies) * a.tiles * a.groups;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int f = u / (a.tiles * a.groups);
    const int rest = u - f * a.tiles * a.groups;
    const int tile = rest / a.groups, grp = rest - tile * a.groups;
    const int* c = a.cpy + (int64_t)f * 3;
    const int src = c[0], dst = c[1], npos = c[2];
    const int e = tile * kK7Threads + threadIdx.x;
    if (e >= npos * a.words_per_pos) continue;
    const int pos = e / a.words_per_pos;
    const int64_t off = pos * a.pos_stride + (int64_t)(e - pos * a.words_per_pos) * WORD;
    const int64_t so = src * a.block_stride + off, d = dst * a.block_stride + off;
    const int p0 = grp * kCopyPlanes;
    const int np = min(kCopyPlanes, a.n_planes - p0);
    WT v[kCopyPlanes];
#pragma unroll
    for (int k = 0; k < kCopyPlanes; ++k)
      if (k < np) v[k] = __builtin_nontemporal_load(reinterpret_cast<const WT*>(a.pools[p0 + k] + so));
#pragma unroll
    for (int k = 0; k < kCopyPlanes; ++k)
      if (k < np) __builtin_nontemporal_store(v[k], reinterpret_cast<WT*>(a.pools[p0 + k] + d));
  }
}

// Reset: row r of item b holds block b*bpi + w in logical block 0; the other
// blocks of the item are free.
__global__ void k6_paged_init(PagedDev pg, int B, int W, int bpi, int mb) {
  const int b = blockIdx.x;
  const int base = b * bpi;
  for (int e = threadIdx.x; e < bpi; e += blockDim.x) {
    pg.refc[base + e] = e < W ? 1 : 0;
    if (e < bpi - W) pg.freel[base + e] = base + bpi - 1 - e;
  }
  for (int e = threadIdx.x; e < W * mb; e += blockDim.x) {
    const int i = e / mb, k = e - i * mb;
    pg.table[(int64_t)b * W * mb + e] = k == 0 ? base + i : -1;
  }
  if (threadIdx.x == 0) {
    pg.nfree[b] = bpi - W;
    if (b == 0) {
      pg.overflow[0] = 0;
      pg.ncpy[0] = 0;
      pg.ncpy[1] = 0;
    }
  }
}

}  // namespace
