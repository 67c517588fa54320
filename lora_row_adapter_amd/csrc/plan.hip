// plan.hip -- the plan step of the LoRA linear layer and the page-table
// translation kernel.
//
// Plan ("Adapter Residency When One Replica Serves Many Fine-Tunes", section
// "Batch composition under many adapters": sort a batch's rows by adapter
// before the forward pass so every adapter's rows are contiguous; "S-LoRA:
// what the paper actually says ...", section "Batched LoRA computation": the
// corrections run as one segmented operation over the adapter-sorted rows).
//
// One workgroup (256 threads up to 1024 rows, else 1024) does the whole plan
// for up to 8192 rows:
//   1. classify each row (none / adapted / bad id / bad rank / bad page) and
//      form the key (adapter << row_bits) | row, or a sentinel for rows that
//      take no adapter;
//   2. bitonic-sort the keys in LDS -- keys are unique, so the order is the
//      stable (adapter, row) order and the result is unique;
//   3. mark segment heads, scan them, and write perm, the segment table and
//      the gather / SGMV work-item lists (segments cut into row blocks).
// Integer atomics only (exact counts); nothing depends on thread timing.
#include "kernels.hpp"

namespace lora {

namespace {

constexpr uint32_t kSentinel = 0xFFFFFFFFu;

// Exclusive scan of one int per thread over an NT-thread block.
// `wsum` is LDS scratch of >= NT / 64 + 1 ints; returns the exclusive prefix
// and writes the block total to *total (every thread sees it).
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *wsum, int *total) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();  // wsum may still be read by a previous scan
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = (lane < NT / 64) ? wsum[lane] : 0;
    int inc = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane < NT / 64) wsum[lane] = inc - w;
    if (lane == NT / 64 - 1) wsum[NT / 64] = inc;
  }
  __syncthreads();
  *total = wsum[NT / 64];
  return x - v + wsum[wave];
}

template <int NT>
__global__ __launch_bounds__(NT) void k_plan(PlanArgs a) {
  // keys [n2] then segment starts [n2] (uint16), sized at launch
  extern __shared__ __attribute__((aligned(16))) uint8_t plan_lds[];
  uint32_t *keys = reinterpret_cast<uint32_t *>(plan_lds);
  uint16_t *sstart = reinterpret_cast<uint16_t *>(plan_lds + ((size_t)4 << a.row_bits));
  __shared__ int wsum[32];
  __shared__ int cnt[4];

  const int tid = threadIdx.x;
  const int M = a.M;
  const int n2 = 1 << a.row_bits;
  int32_t *hdr = reinterpret_cast<int32_t *>(a.ws + a.L.hdr);
  int32_t *perm = reinterpret_cast<int32_t *>(a.ws + a.L.perm);
  int32_t *seg_adapter = reinterpret_cast<int32_t *>(a.ws + a.L.seg_adapter);
  int32_t *seg_start = reinterpret_cast<int32_t *>(a.ws + a.L.seg_start);
  int32_t *seg_len = reinterpret_cast<int32_t *>(a.ws + a.L.seg_len);
  Item *items_g = reinterpret_cast<Item *>(a.ws + a.L.items_g);
  Item *items_s = reinterpret_cast<Item *>(a.ws + a.L.items_s);

  if (tid < 4) cnt[tid] = 0;
  __syncthreads();

  // 1. classify
  for (int m = tid; m < n2; m += NT) {
    uint32_t key = kSentinel;
    if (m < M) {
      const int id = a.ids[m];
      if (id == -1) {
        // no adapter
      } else if (id < -1 || id >= a.S) {
        atomicAdd(&cnt[0], 1);
      } else {
        // every slice's rank must be in range, then every slice's pages
        bool rank_ok = true, page_ok = true;
        for (int q = 0; q < a.n_slices; ++q) {
          const PlanSlice &sl = a.sl[q];
          const int r = sl.ranks[id];
          if (r < 0 || r > sl.R) {
            rank_ok = false;
            continue;
          }
          if (sl.page_table != nullptr) {
            const int64_t bytes = (int64_t)r * sl.bytes_per_rank;
            const int64_t pages = (bytes + sl.page_bytes - 1) / sl.page_bytes;
            if (pages > sl.max_pages) page_ok = false;
            for (int64_t j = 0; page_ok && j < pages; ++j) {
              const int32_t pg = sl.page_table[(int64_t)id * sl.max_pages + j];
              if (pg < 0 || (int64_t)pg >= sl.n_pages) page_ok = false;
            }
          }
        }
        if (!rank_ok) {
          atomicAdd(&cnt[1], 1);
        } else if (!page_ok) {
          atomicAdd(&cnt[2], 1);
        } else {
          key = ((uint32_t)id << a.row_bits) | (uint32_t)m;
          atomicAdd(&cnt[3], 1);
        }
      }
    }
    keys[m] = key;
  }
  __syncthreads();

  // 2. bitonic sort, ascending, n2 keys (n2 a power of two)
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += NT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint32_t ka = keys[lo], kb = keys[hi];
        if ((ka > kb) == up) {
          keys[lo] = kb;
          keys[hi] = ka;
        }
      }
      __syncthreads();
    }
  }

  // 3. segments
  const int n_ad = cnt[3];
  const uint32_t rmask = (1u << a.row_bits) - 1u;
  const int chunk = (n2 + NT - 1) / NT;
  const int i0 = tid * chunk;
  int heads = 0;
  for (int i = i0; i < i0 + chunk; ++i) {
    if (i < n_ad) heads += (i == 0 || (keys[i] >> a.row_bits) != (keys[i - 1] >> a.row_bits));
  }
  int n_seg = 0;
  int run = block_exclusive_scan<NT>(heads, wsum, &n_seg);
  for (int i = i0; i < i0 + chunk; ++i) {
    if (i < n_ad) {
      const bool head = (i == 0 || (keys[i] >> a.row_bits) != (keys[i - 1] >> a.row_bits));
      run += head;
      perm[i] = (int32_t)(keys[i] & rmask);
      if (head) {
        const int s = (int)(keys[i] >> a.row_bits);
        sstart[run - 1] = (uint16_t)i;
        seg_start[run - 1] = i;
        seg_adapter[run - 1] = s;
      }
    }
  }
  __syncthreads();

  // segment lengths and work-item counts
  const int schunk = (n_seg + NT - 1) / NT;
  const int s0 = tid * schunk;
  int ng = 0, ns = 0;
  for (int s = s0; s < s0 + schunk && s < n_seg; ++s) {
    const int len = ((s + 1 < n_seg) ? (int)sstart[s + 1] : n_ad) - (int)sstart[s];
    seg_len[s] = len;
    ng += (len + kRowsPerGatherItem - 1) / kRowsPerGatherItem;
    ns += (len + kRowsPerSgmvItem - 1) / kRowsPerSgmvItem;
  }
  int n_items_g = 0, n_items_s = 0;
  int og = block_exclusive_scan<NT>(ng, wsum, &n_items_g);
  int os = block_exclusive_scan<NT>(ns, wsum, &n_items_s);
  for (int s = s0; s < s0 + schunk && s < n_seg; ++s) {
    const int st = sstart[s];
    const int len = ((s + 1 < n_seg) ? (int)sstart[s + 1] : n_ad) - st;
    const int ad = (int)(keys[st] >> a.row_bits);
    for (int p = 0; p < len; p += kRowsPerGatherItem) {
      Item it;
      it.adapter = ad;
      it.pos = st + p;
      it.nrows = min(kRowsPerGatherItem, len - p);
      it.seg = s;
      items_g[og++] = it;
    }
    for (int p = 0; p < len; p += kRowsPerSgmvItem) {
      Item it;
      it.adapter = ad;
      it.pos = st + p;
      it.nrows = min(kRowsPerSgmvItem, len - p);
      it.seg = s;
      items_s[os++] = it;
    }
  }
  if (tid == 0) {
    hdr[kHdrBadIds] = cnt[0];
    hdr[kHdrBadRanks] = cnt[1];
    hdr[kHdrBadPages] = cnt[2];
    hdr[kHdrAdapted] = n_ad;
    hdr[kHdrSegments] = n_seg;
    hdr[kHdrItemsGather] = n_items_g;
    hdr[kHdrItemsSgmv] = n_items_s;
    hdr[kHdrRows] = M;
  }
}

__global__ __launch_bounds__(256) void k_translate(AdapterRef ar, int32_t S, int64_t n_pages,
                                                   const int32_t *adapter, const int64_t *off,
                                                   int64_t n, int64_t *phys) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t a = adapter[i];
  const int64_t o = off[i];
  int64_t out = -1;
  if (a >= 0 && a < S && o >= 0) {
    const int64_t lp = o >> ar.page_shift;
    if (lp < ar.max_pages) {
      const int64_t p = ar.page_table[(int64_t)a * ar.max_pages + lp];
      if (p >= 0 && p < n_pages) out = (p << ar.page_shift) + (o & (ar.page_bytes - 1));
    }
  }
  phys[i] = out;
}

}  // namespace

hipError_t launch_plan(const PlanArgs &a, hipStream_t st) {
  // LDS sized to the batch (6 bytes per sort slot), so a small plan fits on
  // a CU beside a GEMM workgroup; small batches use fewer waves
  const size_t lds = (size_t)6 << a.row_bits;
  if ((1 << a.row_bits) <= 1024)
    hipLaunchKernelGGL(k_plan<256>, dim3(1), dim3(256), lds, st, a);
  else
    hipLaunchKernelGGL(k_plan<kPlanThreads>, dim3(1), dim3(kPlanThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_translate(const AdapterRef &ar, int32_t S, int64_t n_pages,
                            const int32_t *adapter, const int64_t *off, int64_t n,
                            int64_t *phys, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_translate, dim3((unsigned)blocks), dim3(256), 0, st, ar, S, n_pages,
                     adapter, off, n, phys);
  return hipGetLastError();
}

}  // namespace lora
