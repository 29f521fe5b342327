// gqa_attn.hip - standalone grouped-query decode attention entry point.
// The attention itself is in gqa_attn.h (shared with the decoder step).
#include <atomic>

#include "gqa_attn.h"
#include "vox_host.h"

namespace vox {

// Two resident workgroups per compute unit (at most 128 registers per lane).
// LATE_V (split windows), groups up to 4: at least four waves per SIMD, i.e. two resident workgroups per
// compute unit.
template <int GROUP, bool LATE_V>
__global__ __launch_bounds__(ATTN_THREADS) __attribute__((amdgpu_waves_per_eu(LATE_V && GROUP == 1 ? 4 : LATE_V && GROUP <= 4 ? 2 : 1))) void gqa_attn_kernel(AttnArgs a)
{
    attn_chunk<GROUP, LATE_V>(a);
}

// grid: n_kv_heads * GROUP, one query head per workgroup
template <int GROUP>
__global__ __launch_bounds__(ATTN_MERGE_THREADS) void gqa_attn_merge_kernel(AttnArgs a, int nsplit)
{
    __shared__ AttnMergeLds lds;
    attn_merge<GROUP>(a, blockIdx.x / GROUP, blockIdx.x % GROUP, nsplit, lds);
}

// Up to eight chunks: one workgroup per (query head, chunk), each reading its KV head's chunk
// (the group's heads share it through the cache).  More chunks: one workgroup per (KV head,
// chunk) serving the group's query heads from one load of K and V (measured on MI355X: past
// eight chunks the extra reads of the shared chunks cost more than the spread).  A split window
// ends with the merge.
template <int GROUP>
static int launch_attn(const AttnArgs &a, int n_kv, hipStream_t s)
{
    const AttnPlan plan = attn_plan(a.n_valid, a.s_cap);
    const bool per_head = plan.splits <= 8;
    AttnArgs b = a;
    if (per_head)
        b.kv_shift = GROUP == 8 ? 3 : GROUP == 4 ? 2 : GROUP == 2 ? 1 : 0;
    if (plan.splits == 1)
        hipLaunchKernelGGL((gqa_attn_kernel<1, false>), dim3(1, n_kv * GROUP), dim3(ATTN_THREADS), 0, s, b);
    else if (per_head)
        hipLaunchKernelGGL((gqa_attn_kernel<1, true>), dim3(plan.splits, n_kv * GROUP), dim3(ATTN_THREADS), 0, s, b);
    else
        hipLaunchKernelGGL((gqa_attn_kernel<GROUP, true>), dim3(plan.splits, n_kv), dim3(ATTN_THREADS), 0, s, b);
    int st = check_launch("gqa attention launch");
    if (st || plan.splits == 1)
        return st;
    if (per_head)
        hipLaunchKernelGGL(gqa_attn_merge_kernel<1>, dim3(n_kv * GROUP), dim3(ATTN_MERGE_THREADS), 0, s, b, plan.splits);
    else
        hipLaunchKernelGGL(gqa_attn_merge_kernel<GROUP>, dim3(n_kv * GROUP), dim3(ATTN_MERGE_THREADS), 0, s, b,
                           plan.splits);
    return check_launch("gqa attention merge launch");
}

// Checks every argument but the workspace; returns VOX_OK or a failure status.
static int check_attn_args(const char *who, const float *q, const float *k_cache, const float *v_cache, float *out,
                           int n_q_heads, int n_kv_heads, int head_dim, int n_slots, int n_valid, float scale)
{
    if (!q || !k_cache || !v_cache || !out)
        return fail(VOX_E_INVAL, "%s: null pointer", who);
    if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads)
        return fail(VOX_E_INVAL, "%s: n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", who, n_q_heads,
                    n_kv_heads);
    if (n_slots <= 0 || n_valid < 1 || n_valid > n_slots)
        return fail(VOX_E_INVAL, "%s: need 1 <= n_valid (%d) <= n_slots (%d)", who, n_valid, n_slots);
    if (!(scale == scale))
        return fail(VOX_E_INVAL, "%s: scale is NaN", who);
    const int group = n_q_heads / n_kv_heads;
    if (head_dim != ATTN_HD || (group != 1 && group != 2 && group != 4 && group != 8))
        return fail(VOX_E_UNSUPPORTED, "%s: needs head_dim 128 and a group size in {1,2,4,8}", who);
    if ((int64_t)n_kv_heads * n_slots * head_dim > ((int64_t)1 << 34))
        return fail(VOX_E_UNSUPPORTED, "%s: cache too large", who);
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
        return fail(VOX_E_UNSUPPORTED, "%s: buffers must be 16-byte aligned", who);
    const size_t cache_bytes = (size_t)n_kv_heads * n_slots * head_dim * 4;
    const size_t out_bytes = (size_t)n_q_heads * head_dim * 4;
    if (overlaps(out, out_bytes, q, out_bytes) || overlaps(out, out_bytes, k_cache, cache_bytes) ||
        overlaps(out, out_bytes, v_cache, cache_bytes))
        return fail(VOX_E_INVAL, "%s: output overlaps an input", who);
    return VOX_OK;
}

static int run_attn(const float *q, const float *k_cache, const float *v_cache, float *out, int n_q_heads,
                    int n_kv_heads, int n_slots, int n_valid, float scale, float *part, hipStream_t s)
{
    AttnArgs a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.out = out;
    a.part = part;
    a.pos = nullptr;
    a.n_slots = n_slots;
    a.n_valid = n_valid;
    a.s_cap = attn_split_cap(n_slots);
    a.scale = scale;
    switch (n_q_heads / n_kv_heads) {
    case 1: return launch_attn<1>(a, n_kv_heads, s);
    case 2: return launch_attn<2>(a, n_kv_heads, s);
    case 4: return launch_attn<4>(a, n_kv_heads, s);
    default: return launch_attn<8>(a, n_kv_heads, s);
    }
}

// Split partials of the entry point that allocates nothing: a fixed device array, one copy per
// GPU, which the calls on that GPU share.  Host code never passes `scratch` itself to a kernel
// (on the host it names a stand-in, not device memory); it passes the address that
// hipGetSymbolAddress returned for the current device.
constexpr size_t ATTN_STATIC_SCRATCH_BYTES = (size_t)1 << 20;
static __device__ __align__(256) float scratch[ATTN_STATIC_SCRATCH_BYTES / sizeof(float)];

constexpr int MAX_DEVICES = 64;
static std::atomic<float *> g_scratch_ptr[MAX_DEVICES];

// Device address of `scratch` on the current device (looked up once per device).
static int static_scratch(float **out)
{
    int dev = 0;
    int st = check_hip(hipGetDevice(&dev), "vox_gqa_decode_attn_noalloc: hipGetDevice");
    if (st)
        return st;
    if (dev < 0 || dev >= MAX_DEVICES)
        return fail(VOX_E_UNSUPPORTED, "vox_gqa_decode_attn_noalloc: device ordinal %d beyond %d", dev, MAX_DEVICES);
    float *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        void *sym = nullptr;
        st = check_hip(hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch)), "vox_gqa_decode_attn_noalloc: scratch address");
        if (st)
            return st;
        if (!sym)
            return fail(VOX_E_HIP, "vox_gqa_decode_attn_noalloc: null scratch address");
        p = (float *)sym;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return VOX_OK;
}

}  // namespace vox

using namespace vox;

extern "C" size_t vox_gqa_decode_attn_workspace(int n_q_heads, int n_kv_heads, int head_dim, int n_slots)
{
    if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads || head_dim != ATTN_HD || n_slots <= 0)
        return 0;
    const int group = n_q_heads / n_kv_heads;
    return (size_t)n_kv_heads * attn_split_cap(n_slots) * group * ATTN_PART * sizeof(float);
}

extern "C" int vox_gqa_decode_attn(const float *q, const float *k_cache, const float *v_cache, float *out,
                                   int n_q_heads, int n_kv_heads, int head_dim, int n_slots, int n_valid,
                                   float scale, void *workspace, size_t workspace_bytes, void *stream)
{
    int st = check_attn_args("vox_gqa_decode_attn", q, k_cache, v_cache, out, n_q_heads, n_kv_heads, head_dim, n_slots,
                             n_valid, scale);
    if (st)
        return st;
    if (!workspace)
        return fail(VOX_E_INVAL, "vox_gqa_decode_attn: null workspace");
    if (!aligned(workspace, 16))
        return fail(VOX_E_UNSUPPORTED, "vox_gqa_decode_attn: workspace must be 16-byte aligned");
    const size_t need = vox_gqa_decode_attn_workspace(n_q_heads, n_kv_heads, head_dim, n_slots);
    if (workspace_bytes < need)
        return fail(VOX_E_WORKSPACE, "vox_gqa_decode_attn: workspace %zu bytes, need %zu", workspace_bytes, need);
    const size_t cache_bytes = (size_t)n_kv_heads * n_slots * head_dim * 4;
    const size_t out_bytes = (size_t)n_q_heads * head_dim * 4;
    if (overlaps(workspace, need, out, out_bytes) || overlaps(workspace, need, q, out_bytes) ||
        overlaps(workspace, need, k_cache, cache_bytes) || overlaps(workspace, need, v_cache, cache_bytes))
        return fail(VOX_E_INVAL, "vox_gqa_decode_attn: workspace overlaps another buffer");
    st = run_attn(q, k_cache, v_cache, out, n_q_heads, n_kv_heads, n_slots, n_valid, scale, (float *)workspace,
                  (hipStream_t)stream);
    return st ? st : ok();
}

extern "C" int vox_gqa_decode_attn_noalloc(const float *q, const float *k_cache, const float *v_cache, float *out,
                                          int n_q_heads, int n_kv_heads, int head_dim, int n_slots, int n_valid,
                                          float scale, void *stream)
{
    int st = check_attn_args("vox_gqa_decode_attn_noalloc", q, k_cache, v_cache, out, n_q_heads, n_kv_heads, head_dim,
                             n_slots, n_valid, scale);
    if (st)
        return st;
    const size_t need = vox_gqa_decode_attn_workspace(n_q_heads, n_kv_heads, head_dim, n_slots);
    if (need > ATTN_STATIC_SCRATCH_BYTES)
        return fail(VOX_E_UNSUPPORTED,
                    "vox_gqa_decode_attn_noalloc: %zu bytes of split partials exceed the fixed %zu-byte scratch "
                    "(n_q_heads * min(32, ceil(n_slots / 128)) * 528 bytes)",
                    need, ATTN_STATIC_SCRATCH_BYTES);
    float *part = nullptr;
    st = static_scratch(&part);
    if (st)
        return st;
    st = run_attn(q, k_cache, v_cache, out, n_q_heads, n_kv_heads, n_slots, n_valid, scale, part,
                  (hipStream_t)stream);
    return st ? st : ok();
}
