// KMCU v1 container reader (host side of the boundary).
//
// Minueza-32M -> KMCU v1 page (pnsm.cn/news/1981961.html), section 4: a
// 128-byte little-endian header (magic "KMCU", u32 version 1, the model's
// u32 sizes and ids, n_tensors, dir_offset, data_offset, f32 rope_theta and
// norm_eps, u32 total_params), n_tensors 48-byte directory records (24-byte
// name, u8 dtype at byte 24: 1 = f32, 2 = Q4_0; u32 n_rows, n_cols, absolute
// offset and nbytes at bytes 28..43), tensor data 64-byte aligned.
//
// The reader works on the file's bytes where the caller holds them (read or
// mapped into host memory) and validates every field it hands out against
// the file: nothing is parsed twice and no tensor is copied until
// kmcu_upload moves one into a device buffer the caller owns.
#include <cstring>

#include "bqm_common.h"

namespace bqm {
namespace {

constexpr uint64_t kHeaderBytes = 128, kRecordBytes = 48, kAlign = 64;

uint32_t u32_at(const uint8_t *p, uint64_t off) {
  uint32_t v;
  memcpy(&v, p + off, 4);                          // little-endian host (x86-64)
  return v;
}

float f32_at(const uint8_t *p, uint64_t off) {
  float v;
  memcpy(&v, p + off, 4);
  return v;
}

uint64_t payload_bytes(uint32_t dtype, uint32_t rows, uint32_t cols) {
  if (dtype == BQM_KMCU_F32) return (uint64_t)rows * cols * 4;
  return (uint64_t)rows * (((uint64_t)cols + 31) / 32) * 18;   // Q4_0: 18-byte blocks, rows padded to 32
}

}  // namespace
}  // namespace bqm

using namespace bqm;

extern "C" {

int kmcu_header(const void *file, uint64_t size, bqm_kmcu_header *h) {
  if (!file || !h) return BQM_EINVAL;
  const uint8_t *p = static_cast<const uint8_t *>(file);
  if (size < kHeaderBytes || memcmp(p, "KMCU", 4) != 0) return BQM_EINVAL;
  bqm_kmcu_header o;
  o.version = u32_at(p, 4);
  o.n_layers = u32_at(p, 8);
  o.dim = u32_at(p, 12);
  o.n_heads = u32_at(p, 16);
  o.n_kv_heads = u32_at(p, 20);
  o.head_dim = u32_at(p, 24);
  o.ffn_dim = u32_at(p, 28);
  o.vocab_size = u32_at(p, 32);
  o.max_seq = u32_at(p, 36);
  o.bos_id = u32_at(p, 40);
  o.eos_id = u32_at(p, 44);
  o.tied_embed = u32_at(p, 48);
  o.n_tensors = u32_at(p, 52);
  o.dir_offset = u32_at(p, 56);
  o.data_offset = u32_at(p, 60);
  o.rope_theta = f32_at(p, 64);
  o.norm_eps = f32_at(p, 68);
  o.total_params = u32_at(p, 72);
  if (o.version != 1) return BQM_ENOTSUP;
  if (o.dir_offset < kHeaderBytes || (uint64_t)o.dir_offset + (uint64_t)o.n_tensors * kRecordBytes > size ||
      o.data_offset > size || o.data_offset % kAlign != 0)
    return BQM_EINVAL;
  *h = o;
  return BQM_OK;
}

int kmcu_tensor(const void *file, uint64_t size, int index, bqm_kmcu_tensor *t) {
  if (!t) return BQM_EINVAL;
  bqm_kmcu_header h;
  const int rc = kmcu_header(file, size, &h);
  if (rc) return rc;
  if (index < 0 || (uint32_t)index >= h.n_tensors) return BQM_EINVAL;
  const uint8_t *p = static_cast<const uint8_t *>(file);
  const uint64_t rec = (uint64_t)h.dir_offset + (uint64_t)index * kRecordBytes;
  bqm_kmcu_tensor o;
  memset(&o, 0, sizeof(o));
  memcpy(o.name, p + rec, 24);                     // zero-padded; o.name[24] stays 0
  o.dtype = p[rec + 24];
  o.n_rows = u32_at(p, rec + 28);
  o.n_cols = u32_at(p, rec + 32);
  o.offset = u32_at(p, rec + 36);
  o.nbytes = u32_at(p, rec + 40);
  if (o.dtype != BQM_KMCU_F32 && o.dtype != BQM_KMCU_Q4) return BQM_EINVAL;
  if (o.n_rows == 0 || o.n_cols == 0) return BQM_EINVAL;
  if (o.nbytes != payload_bytes(o.dtype, o.n_rows, o.n_cols)) return BQM_EINVAL;
  if (o.offset % kAlign != 0 || o.offset < h.data_offset || (uint64_t)o.offset + o.nbytes > size)
    return BQM_EINVAL;
  *t = o;
  return BQM_OK;
}

int kmcu_find(const void *file, uint64_t size, const char *name, bqm_kmcu_tensor *t) {
  if (!name || !t) return BQM_EINVAL;
  bqm_kmcu_header h;
  int rc = kmcu_header(file, size, &h);
  if (rc) return rc;
  for (uint32_t i = 0; i < h.n_tensors; ++i) {
    bqm_kmcu_tensor c;
    rc = kmcu_tensor(file, size, (int)i, &c);
    if (rc) return rc;
    if (strncmp(c.name, name, 25) == 0) {
      *t = c;
      return BQM_OK;
    }
  }
  return BQM_EINVAL;
}

int kmcu_upload(const void *file, uint64_t size, const bqm_kmcu_tensor *t, void *dst,
                bqm_stream_t stream) {
  if (!file || !t || !dst) return BQM_EINVAL;
  // the record may come from the caller: the same checks as kmcu_tensor's
  if ((t->dtype != BQM_KMCU_F32 && t->dtype != BQM_KMCU_Q4) || t->n_rows == 0 || t->n_cols == 0 ||
      (uint64_t)t->offset + t->nbytes > size || t->offset % kAlign != 0 ||
      t->nbytes != payload_bytes(t->dtype, t->n_rows, t->n_cols))
    return BQM_EINVAL;
  if (((uintptr_t)dst & 15u) != 0) return BQM_EALIGN;
  const hipError_t e = hipMemcpyAsync(dst, static_cast<const uint8_t *>(file) + t->offset, t->nbytes,
                                      hipMemcpyHostToDevice, (hipStream_t)stream);
  return e == hipSuccess ? BQM_OK : BQM_EDEVICE;
}

int kmcu_upload_data(const void *file, uint64_t size, void *dst, uint64_t dst_bytes, bqm_stream_t stream) {
  if (!dst) return BQM_EINVAL;
  bqm_kmcu_header h;
  int rc = kmcu_header(file, size, &h);
  if (rc) return rc;
  for (uint32_t i = 0; i < h.n_tensors; ++i) {     // every record in range before anything moves
    bqm_kmcu_tensor t;
    rc = kmcu_tensor(file, size, (int)i, &t);
    if (rc) return rc;
  }
  const uint64_t n = size - h.data_offset;
  if (dst_bytes < n) return BQM_EINVAL;
  if (((uintptr_t)dst & 15u) != 0) return BQM_EALIGN;
  if (n == 0) return BQM_OK;
  const hipError_t e = hipMemcpyAsync(dst, static_cast<const uint8_t *>(file) + h.data_offset, n,
                                      hipMemcpyHostToDevice, (hipStream_t)stream);
  return e == hipSuccess ? BQM_OK : BQM_EDEVICE;
}

}  // extern "C"
