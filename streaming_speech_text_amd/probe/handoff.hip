// handoff.hip - grid-wide handoff probe: what a persistent kernel pays to pass a vector between
// phases, against one kernel launch per phase.
//
// Not an operation of the decoder.  It measures the design question of the decoder step (a
// token is a chain of phases - QKV, attention, O, gate/up, down - each needing the whole output
// vector of the one before): can one persistent kernel per layer, with a grid barrier between
// phases and the next phase's weights prefetched before the barrier, beat one launch per phase?
//
// Each phase, every workgroup (one per compute unit, 512 threads): moves its prefetched weight
// share (NCH 16-byte chunks per thread) to LDS, issues the loads of the next phase's share, reads
// the previous phase's 3072-float vector written by the whole grid (agent-scope loads; every value
// checked), folds the staged weights, writes its 12 floats of this phase's vector (agent-scope
// stores), then waits at the grid barrier.  The vectors are double-buffered by phase parity.
// Barriers: mode 0 - every workgroup stores its own flag, workgroup 0 gathers them and releases
// the grid with one flag; mode 1 - eight counters (workgroup i adds to counter i % 8), every
// workgroup polls their sum; mode 2 - the eight counters polled by a ninth wave that holds no
// weight loads, so the working waves keep the next phase's loads in flight across the barrier.
// Every wait is bounded; one expired wait sets an abort flag that
// ends all others, so every workgroup exits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vox_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int HT = 512;                       // threads per workgroup
constexpr int HVEC = 3072;                    // vector length
constexpr size_t OFF_CTL = 0;                 // {abort, timeouts, mismatches, sink}
constexpr size_t OFF_COUNTERS = 256;          // 8 counters, 256 bytes apart
constexpr size_t OFF_RELEASE = 4096;
constexpr size_t OFF_FLAGS = 8192;            // one flag per workgroup, 64 bytes apart
constexpr int MAX_WG = 4096;
constexpr size_t OFF_VEC = OFF_FLAGS + (size_t)MAX_WG * 64;
constexpr size_t WORK_BYTES = OFF_VEC + 2 * HVEC * 4 + 4096;
constexpr unsigned SPIN_LIMIT = 1u << 20;     // polls before a wait gives up

struct Ctl {
    unsigned abort_flag, timeouts, mismatches, sink;
};

struct Work {
    Ctl *ctl;
    unsigned *counters, *release, *flags;
    float *vec;
};

__device__ __forceinline__ Work work_of(uint8_t *w)
{
    return Work{(Ctl *)(w + OFF_CTL), (unsigned *)(w + OFF_COUNTERS), (unsigned *)(w + OFF_RELEASE),
                (unsigned *)(w + OFF_FLAGS), (float *)(w + OFF_VEC)};
}

__device__ __forceinline__ void st_agent(unsigned *p, unsigned v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_agent(const unsigned *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void zero_kernel(uint32_t *w, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        w[i] = 0u;
}

// Gives up a wait: records it and raises the abort flag that ends every other wait.
__device__ void give_up(const Work &W, int lane)
{
    if (lane == 0) {
        st_agent(&W.ctl->abort_flag, 1u);
        __hip_atomic_fetch_add(&W.ctl->timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int MODE>
__device__ void grid_barrier(const Work &W, int p)
{
    const int G = gridDim.x;
    const int lane = threadIdx.x & 63;
    __builtin_amdgcn_s_waitcnt(0);   // this workgroup's vector stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        if (MODE == 0)
            st_agent(W.flags + blockIdx.x * 16, (unsigned)p);
        else
            __hip_atomic_fetch_add(W.counters + (blockIdx.x & 7) * 64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x < 64) {
        unsigned n = 0;
        if (MODE == 0 && blockIdx.x == 0) {
            for (;;) {
                bool ok = true;
                for (int j = lane; j < G; j += 64)
                    ok = ok && ld_agent(W.flags + j * 16) >= (unsigned)p;
                if (__all(ok))
                    break;
                if (++n > SPIN_LIMIT || ld_agent(&W.ctl->abort_flag)) {
                    give_up(W, lane);
                    break;
                }
            }
            if (lane == 0)
                st_agent(W.release, (unsigned)p);
        } else {
            for (;;) {
                bool ok;
                if (MODE == 0) {
                    ok = ld_agent(W.release) >= (unsigned)p;
                } else {
                    unsigned c = lane < 8 ? ld_agent(W.counters + lane * 64) : 0u;
                    c += __shfl_xor(c, 1);
                    c += __shfl_xor(c, 2);
                    c += __shfl_xor(c, 4);
                    ok = __shfl(c, 0) >= (unsigned)p * (unsigned)G;
                }
                if (ok)
                    break;
                if (++n > SPIN_LIMIT || ld_agent(&W.ctl->abort_flag)) {
                    give_up(W, lane);
                    break;
                }
            }
        }
    }
    __syncthreads();
}

// Checks the previous phase's vector (written by every workgroup) and returns a fold of it.
__device__ float read_vector(const Work &W, int p, bool agent_scope)
{
    const int per = HVEC / gridDim.x;
    const float *v = W.vec + (size_t)((p - 1) & 1) * HVEC;
    float s = 0.0f;
    for (int i = threadIdx.x; i < per * (int)gridDim.x; i += HT) {
        const float x = agent_scope ? __hip_atomic_load(v + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : v[i];
        if (x != (float)((p - 1) * 4096 + i / per))
            __hip_atomic_fetch_add(&W.ctl->mismatches, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s += x;
    }
    return s;
}

template <int MODE, int NCH>
__global__ __launch_bounds__(HT) void handoff_persistent_kernel(const u32x4 *__restrict__ wts, int64_t win16, int nwin,
                                                                uint8_t *work, int nphase)
{
    __shared__ u32x4 lds[NCH > 0 ? NCH * HT : 1];
    const Work W = work_of(work);
    const int per = HVEC / gridDim.x;
    u32x4 pf[NCH > 0 ? NCH : 1];
    u32x4 acc = {0u, 0u, 0u, 0u};
    auto issue = [&](int p) {
        const u32x4 *base = wts + (int64_t)(p % nwin) * win16 + (int64_t)blockIdx.x * NCH * HT;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            pf[c] = base[c * HT + threadIdx.x];
    };
    if constexpr (NCH > 0)
        issue(1);
    for (int p = 1; p <= nphase; ++p) {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            lds[c * HT + threadIdx.x] = pf[c];
        if (NCH > 0 && p < nphase)
            issue(p + 1);
        const float s = p > 1 ? read_vector(W, p, true) : 0.0f;
        __syncthreads();
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            acc ^= lds[((c + 1) % (NCH > 0 ? NCH : 1)) * HT + threadIdx.x];
        if ((int)threadIdx.x < per)
            __hip_atomic_store(W.vec + (size_t)(p & 1) * HVEC + blockIdx.x * per + threadIdx.x,
                               (float)(p * 4096 + (int)blockIdx.x) + 0.0f * s, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        grid_barrier<MODE>(W, p);
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u)
        atomicAdd(&W.ctl->sink, 1u);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int WAIT_LGKM0 = 0xC07F;   // LDS and scalar memory done; vector memory untouched
constexpr int WAIT_ALL0 = 0;         // everything done

// Mode 2: the same phases with the next phase's weight loads in flight across the barrier.  A
// ninth wave in each workgroup keeps no weight loads: it stores the workgroup's share of the
// phase's vector (agent scope), waits for its own stores, adds the workgroup to the eight
// counters, polls their sum, reads the grid's vector for the next phase (agent scope) into LDS,
// and releases the eight working waves.  Those check every value of that vector, fold their
// prefetched weights, hand their share of the next vector to the poller through LDS, issue the
// next phase's loads and wait
// at workgroup barriers that wait on no memory, so their loads stay in flight while the grid
// synchronises (memory returns in order per wave: the poller's loads never queue behind them).
template <int NCH>
__global__ __launch_bounds__(HT + 64) void handoff_poller_kernel(const u32x4 *__restrict__ wts, int64_t win16, int nwin,
                                                                 uint8_t *work, int nphase)
{
    __shared__ float vin[HVEC];   // the previous phase's vector
    __shared__ float vout[64];    // this workgroup's share of the phase's vector
    const Work W = work_of(work);
    const int G = gridDim.x;
    const int per = HVEC / G;
    const int tid = threadIdx.x;
    const bool poller = tid >= HT;
    const int lane = tid & 63;
    u32x4 pf[NCH > 0 ? NCH : 1];
    u32x4 acc = {0u, 0u, 0u, 0u};
    auto issue = [&](int p) {
        const u32x4 *base = wts + (int64_t)(p % nwin) * win16 + (int64_t)blockIdx.x * NCH * HT;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            pf[c] = base[c * HT + tid];
    };
    if (!poller && NCH > 0)
        issue(1);
    for (int p = 1; p <= nphase; ++p) {
        if (!poller) {
            float sum = 0.0f;
            if (p > 1) {
                unsigned bad = 0;   // values the poller read before they were visible
                for (int i = tid; i < HVEC; i += HT) {
                    bad += vin[i] != (float)((p - 1) * 4096 + i / per);
                    sum += vin[i];
                }
                if (bad)
                    __hip_atomic_fetch_add(&W.ctl->mismatches, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                acc ^= pf[c];
            if (tid < per)
                vout[tid] = (float)(p * 4096 + (int)blockIdx.x) + 0.0f * sum;
            if constexpr (NCH > 0)
                issue(p + 1);   // in flight until the next phase folds it (past the last phase: unused)
        }
        __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);   // vout written
        __builtin_amdgcn_s_barrier();
        if (poller) {
            if (lane < per)
                __hip_atomic_store(W.vec + (size_t)(p & 1) * HVEC + blockIdx.x * per + lane, vout[lane], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(WAIT_ALL0);   // the poller's stores are complete (it has no loads in flight)
            if (lane == 0)
                __hip_atomic_fetch_add(W.counters + (blockIdx.x & 7) * 64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            unsigned n = 0;
            for (;;) {
                unsigned c = lane < 8 ? ld_agent(W.counters + lane * 64) : 0u;
                c += __shfl_xor(c, 1);
                c += __shfl_xor(c, 2);
                c += __shfl_xor(c, 4);
                if (__shfl(c, 0) >= (unsigned)p * (unsigned)G)
                    break;
                if (++n > SPIN_LIMIT || ld_agent(&W.ctl->abort_flag)) {
                    give_up(W, lane);
                    break;
                }
            }
            if (p < nphase) {
                // a lane's 48 loads all issued before the first is used: one memory round trip
                const float *v = W.vec + (size_t)(p & 1) * HVEC + lane;
                float xs[HVEC / 64];
#pragma unroll
                for (int j = 0; j < HVEC / 64; ++j)
                    xs[j] = __hip_atomic_load(v + 64 * j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                for (int j = 0; j < HVEC / 64; ++j)
                    vin[lane + 64 * j] = xs[j];
            }
        }
        __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);   // vin written
        __builtin_amdgcn_s_barrier();
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u)
        atomicAdd(&W.ctl->sink, 1u);
}

// One phase as its own launch (the same work, without a prefetch or a barrier).
template <int NCH>
__global__ __launch_bounds__(HT) void handoff_phase_kernel(const u32x4 *__restrict__ wts, int64_t win16, int nwin,
                                                           uint8_t *work, int p)
{
    const Work W = work_of(work);
    const int per = HVEC / gridDim.x;
    u32x4 pf[NCH > 0 ? NCH : 1];
    u32x4 acc = {0u, 0u, 0u, 0u};
    const u32x4 *base = wts + (int64_t)(p % nwin) * win16 + (int64_t)blockIdx.x * NCH * HT;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        pf[c] = base[c * HT + threadIdx.x];
    const float s = p > 1 ? read_vector(W, p, false) : 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        acc ^= pf[c];
    if ((int)threadIdx.x < per)
        W.vec[(size_t)(p & 1) * HVEC + blockIdx.x * per + threadIdx.x] = (float)(p * 4096 + (int)blockIdx.x) + 0.0f * s;
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u)
        atomicAdd(&W.ctl->sink, 1u);
}

int grid_size()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1 ||
        cus > MAX_WG)
        return -1;
    return cus;
}

// Window of one phase (bytes) and the number of windows the weight buffer holds.
bool windows(int nch, int G, size_t weight_bytes, int64_t &win16, int &nwin)
{
    const size_t win = (size_t)nch * HT * 16 * G;
    if (nch == 0) {
        win16 = 1;
        nwin = 1;
        return true;
    }
    if (weight_bytes < win)
        return false;
    win16 = (int64_t)(win / 16);
    const size_t n = weight_bytes / win;
    nwin = (int)(n > 1000 ? 1000 : n);
    return true;
}

template <int NCH>
int launch_persistent(int mode, const void *w, int64_t win16, int nwin, void *work, int nphase, int G, hipStream_t s)
{
    int occ = 0;
    const bool fits = mode == 0   ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, handoff_persistent_kernel<0, NCH>, HT, 0) == hipSuccess
                      : mode == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, handoff_persistent_kernel<1, NCH>, HT, 0) == hipSuccess
                                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, handoff_poller_kernel<NCH>, HT + 64, 0) == hipSuccess;
    if (!fits || occ < 1)
        return -2;   // one workgroup per compute unit must be resident at once
    if (mode == 2)
        hipLaunchKernelGGL((handoff_poller_kernel<NCH>), dim3(G), dim3(HT + 64), 0, s, (const u32x4 *)w, win16, nwin,
                           (uint8_t *)work, nphase);
    else if (mode == 0)
        hipLaunchKernelGGL((handoff_persistent_kernel<0, NCH>), dim3(G), dim3(HT), 0, s, (const u32x4 *)w, win16, nwin,
                           (uint8_t *)work, nphase);
    else
        hipLaunchKernelGGL((handoff_persistent_kernel<1, NCH>), dim3(G), dim3(HT), 0, s, (const u32x4 *)w, win16, nwin,
                           (uint8_t *)work, nphase);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace

extern "C" size_t vox_probe_handoff_work_bytes(void) { return WORK_BYTES; }

extern "C" int vox_probe_handoff_reset(void *work, void *stream)
{
    if (!work || (uintptr_t)work % 256)
        return -1;
    hipLaunchKernelGGL(zero_kernel, dim3(64), dim3(256), 0, (hipStream_t)stream, (uint32_t *)work, (int)(WORK_BYTES / 4));
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int vox_probe_handoff_persistent(int mode, int nch, int nphase, const void *weights, size_t weight_bytes,
                                            void *work, void *stream)
{
    const int G = grid_size();
    int64_t win16 = 0;
    int nwin = 0;
    if ((mode != 0 && mode != 1 && mode != 2) || nphase < 1 || nphase > 100000 || !work || (uintptr_t)work % 256 || G < 1 ||
        (nch > 0 && (!weights || (uintptr_t)weights % 16)) || !windows(nch, G, weight_bytes, win16, nwin) ||
        (mode == 2 && (HVEC % G || HVEC / G > 64)))   // the poller stores a share of at most 64 values
        return -1;
    hipStream_t s = (hipStream_t)stream;
    switch (nch) {
    case 0: return launch_persistent<0>(mode, weights, win16, nwin, work, nphase, G, s);
    case 4: return launch_persistent<4>(mode, weights, win16, nwin, work, nphase, G, s);
    case 8: return launch_persistent<8>(mode, weights, win16, nwin, work, nphase, G, s);
    case 16: return launch_persistent<16>(mode, weights, win16, nwin, work, nphase, G, s);
    default: return -1;
    }
}

extern "C" int vox_probe_handoff_phase(int nch, int phase, const void *weights, size_t weight_bytes, void *work,
                                       void *stream)
{
    const int G = grid_size();
    int64_t win16 = 0;
    int nwin = 0;
    if (phase < 1 || phase > 100000 || !work || (uintptr_t)work % 256 || G < 1 ||
        (nch > 0 && (!weights || (uintptr_t)weights % 16)) || !windows(nch, G, weight_bytes, win16, nwin))
        return -1;
    hipStream_t s = (hipStream_t)stream;
    const u32x4 *w = (const u32x4 *)weights;
    switch (nch) {
    case 0: hipLaunchKernelGGL(handoff_phase_kernel<0>, dim3(G), dim3(HT), 0, s, w, win16, nwin, (uint8_t *)work, phase); break;
    case 4: hipLaunchKernelGGL(handoff_phase_kernel<4>, dim3(G), dim3(HT), 0, s, w, win16, nwin, (uint8_t *)work, phase); break;
    case 8: hipLaunchKernelGGL(handoff_phase_kernel<8>, dim3(G), dim3(HT), 0, s, w, win16, nwin, (uint8_t *)work, phase); break;
    case 16: hipLaunchKernelGGL(handoff_phase_kernel<16>, dim3(G), dim3(HT), 0, s, w, win16, nwin, (uint8_t *)work, phase); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
