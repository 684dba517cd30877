// ZeRO-Offload on one GPU and its host ("ZeRO 优化器：把显存“分”着用", ZeRO-Offload: gradients go to
// the CPU asynchronously, the CPU updates the optimizer state, the updated parameters go back to the
// GPU, and a pipeline keeps CPU and GPU working at once).
//
// zero_offload_step runs the whole offloaded step for a rank's shard in chunks, double-buffered:
// the GPU sums the gradient replicas of chunk c+1 and copies it to pinned host memory (or, with no
// device staging, the reduce kernel writes it there itself) while the host updates chunk c
// (zero_host_adam.cpp), and chunk c's 16-bit parameters are copied back to the rank's slot on a
// second stream while the host works on chunk c+1. The host threads are started once per call and
// serve every chunk.
#include <hip/hip_runtime_api.h>

#include "zero_host_adam.h"

extern "C" {

zero_status zero_offload_step(const zero_grad_src* src, uint64_t n, float grad_scale,
                              float* h_master, float* h_m, float* h_v, const zero_adam_hparams* hp,
                              void* d_out_param, int32_t out_dtype,
                              const zero_offload_buffers* buf, void* stream) {
  const char* fn = "zero_offload_step";
  zero_adam_scalars k;
  // the 16-bit slot is device memory: only its dtype is checked here, not host aliasing
  zero_status s = zero::check_host_args(fn, false, nullptr, n, h_master, h_m, h_v, hp, nullptr, out_dtype, &k);
  if (s == ZERO_OK && out_dtype != ZERO_BF16 && out_dtype != ZERO_F16)
    s = zero::fail(out_dtype == ZERO_F32 ? ZERO_E_UNSUPPORTED : ZERO_E_INVAL,
                   "%s: out dtype %d is not bf16 or fp16", fn, out_dtype);
  if (s != ZERO_OK) return s;
  if (!src || !buf) return zero::fail(ZERO_E_INVAL, "%s: NULL source or buffers", fn);
  if (n == 0) return zero::ok();
  if (!d_out_param) return zero::fail(ZERO_E_INVAL, "%s: the parameter slot is NULL", fn);
  if (!buf->h_grad || !buf->h_param || buf->chunk_elems == 0)
    return zero::fail(ZERO_E_INVAL, "%s: incomplete staging buffers", fn);
  for (int a = 0; a < 4; ++a) {
    if (!buf->events[a]) return zero::fail(ZERO_E_INVAL, "%s: event %d is NULL", fn, a);
    for (int b = 0; b < a; ++b)
      if (buf->events[a] == buf->events[b])
        return zero::fail(ZERO_E_INVAL, "%s: events %d and %d are the same", fn, b, a);
  }
  const uint64_t C = buf->chunk_elems;
  if (C > UINT64_MAX / 16) return zero::fail(ZERO_E_OVERFLOW, "%s: chunk too large", fn);
  const int rb = (int)zero::dtype_bytes(src->dtype);
  if (!src->ptrs || src->count == 0 || src->count > ZERO_MAX_REPLICAS)
    return zero::fail(ZERO_E_INVAL, "%s: bad gradient source", fn);
  // where the reduce kernel writes: the device staging, else the pinned host chunks themselves
  const bool direct = buf->d_grad == nullptr;
  float* red = direct ? buf->h_grad : buf->d_grad;
  if (zero::overlaps(d_out_param, n * 2, red, 2 * C * 4))
    return zero::fail(ZERO_E_INVAL, "%s: the slot overlaps the gradient staging", fn);
  for (uint32_t r = 0; r < src->count; ++r) {
    if (zero::overlaps(d_out_param, n * 2, src->ptrs[r], n * rb))
      return zero::fail(ZERO_E_INVAL, "%s: the slot overlaps replica %u", fn, r);
    if (zero::overlaps(red, 2 * C * 4, src->ptrs[r], n * rb))
      return zero::fail(ZERO_E_INVAL, "%s: the gradient staging overlaps replica %u", fn, r);
  }
  if (direct) {
    // The reduce kernel writes h_grad itself: it must be pinned host memory that the device sees at
    // the same address (pageable memory would fault the kernel). Both ends of the range are asked.
    const char* ends[2] = {reinterpret_cast<const char*>(buf->h_grad),
                           reinterpret_cast<const char*>(buf->h_grad + 2 * C) - 1};
    for (const char* p : ends) {
      hipPointerAttribute_t a{};
      const hipError_t pe = hipPointerGetAttributes(&a, p);
      if (pe != hipSuccess) (void)hipGetLastError();   // clear only the error this query set
      if (pe != hipSuccess || a.type != hipMemoryTypeHost || a.devicePointer != p)
        return zero::fail(ZERO_E_INVAL, "%s: with no device staging, h_grad[0, 2 * chunk_elems) must "
                          "be pinned host memory mapped for the device (hipHostMalloc)", fn);
    }
  }

  hipStream_t main = static_cast<hipStream_t>(stream);
  hipStream_t back = buf->h2d_stream ? static_cast<hipStream_t>(buf->h2d_stream) : main;
  // the caller's events: a chunk's gradient has arrived (got), its parameters have left (sent)
  hipEvent_t got[2] = {static_cast<hipEvent_t>(buf->events[0]), static_cast<hipEvent_t>(buf->events[1])};
  hipEvent_t sent[2] = {static_cast<hipEvent_t>(buf->events[2]), static_cast<hipEvent_t>(buf->events[3])};
  hipError_t e = hipSuccess;
  const bool l2 = hp->wd_mode == ZERO_ADAM_L2;
  const uint64_t nchunks = (n + C - 1) / C;
  // one team of host threads for every chunk of this call (threads that cannot start are left out)
  zero::HostTeam team(buf->threads);
  const void* ptrs[ZERO_MAX_REPLICAS];   // one chunk's replica pointers (no allocation)
  bool sent_any[2] = {false, false};

  // enqueue chunk c on the GPU: replica sum into d_grad[b] and a copy to h_grad[b], or the sum
  // straight into h_grad[b]
  auto issue = [&](uint64_t c) -> zero_status {
    const uint64_t off = c * C, len = n - off < C ? n - off : C;
    const int b = (int)(c & 1);
    for (uint32_t r = 0; r < src->count; ++r)
      ptrs[r] = static_cast<const char*>(src->ptrs[r]) + off * rb;
    const zero_grad_src part{ptrs, src->count, src->dtype};
    zero_status rs = zero_reduce_shard(&part, len, red + b * C, nullptr, nullptr, 1.0, main);
    if (rs != ZERO_OK) return rs;
    hipError_t ce = hipSuccess;
    if (!direct)
      ce = hipMemcpyAsync(buf->h_grad + b * C, buf->d_grad + b * C, len * 4, hipMemcpyDeviceToHost,
                          main);
    if (ce == hipSuccess) ce = hipEventRecord(got[b], main);
    if (ce != hipSuccess) return zero::fail(ZERO_E_HIP, "%s: %s", fn, hipGetErrorString(ce));
    return ZERO_OK;
  };

  if (e == hipSuccess) s = issue(0);
  for (uint64_t c = 0; e == hipSuccess && s == ZERO_OK && c < nchunks; ++c) {
    const uint64_t off = c * C, len = n - off < C ? n - off : C;
    const int b = (int)(c & 1);
    if (c + 1 < nchunks) {
      s = issue(c + 1);
      if (s != ZERO_OK) break;
    }
    e = hipEventSynchronize(got[b]);                   // chunk c's gradient is in host memory
    if (e == hipSuccess && sent_any[b]) e = hipEventSynchronize(sent[b]);  // h_param[b] is free
    if (e != hipSuccess) break;
    uint16_t* hp16 = static_cast<uint16_t*>(buf->h_param) + b * C;
    zero::host_step(buf->h_grad + b * C, len, grad_scale, h_master + off, h_m + off, h_v + off, k, l2,
                    hp16, out_dtype, buf->threads, &team);
    e = hipMemcpyAsync(static_cast<uint16_t*>(d_out_param) + off, hp16, len * 2,
                       hipMemcpyHostToDevice, back);
    if (e == hipSuccess) e = hipEventRecord(sent[b], back);
    sent_any[b] = true;
  }
  // the call returns once every parameter copy has landed (the host buffers are then free)
  for (int b = 0; b < 2; ++b) {
    if (sent_any[b] && e == hipSuccess) e = hipEventSynchronize(sent[b]);
  }
  if (e != hipSuccess || s != ZERO_OK) {
    // after a failure, still wait for whatever was enqueued (a gradient copy or the reduce kernel
    // writing h_grad, a parameter copy from h_param), so that nothing touches the caller's host
    // buffers after return
    (void)hipStreamSynchronize(main);
    if (back != main) (void)hipStreamSynchronize(back);
  }
  if (s != ZERO_OK) return s;
  if (e != hipSuccess) return zero::fail(ZERO_E_HIP, "%s: %s", fn, hipGetErrorString(e));
  return zero::ok();
}

}  // extern "C"
