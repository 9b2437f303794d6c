// io.hip -- checkpoint files, token files and the host random number generator of the C ABI
// (include/gpt2.h), written from "llm.c 的中文注解-20240421":
//  - checkpoint: section 1.22 gpt2_build_from_checkpoint -- a header of 256 int32 (magic
//    20240326, version 1, maxT, V, L, NH, C; the rest unused, written as zero), then the
//    fp32 parameters in the order and shapes of section 1.16;
//  - token files: sections 1.28 - 1.32 (DataLoader) -- a flat file of int32 tokens read in
//    windows of B*T+1, inputs = window[0, BT), targets = window[1, BT+1), the window
//    advancing by B*T and going back to the start when the next one would pass the end;
//  - sections 1.33, 1.34: the xorshift* generator and the float in [0, 1) built from it.
// Host code only; device copies go through the HIP runtime.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gpt2.h"
#include "kernels.h"

namespace {

constexpr int32_t kMagic = 20240326;
constexpr int32_t kVersion = 1;
constexpr int kHeaderInts = 256;

int io_fail(int code, const char* fmt, const char* path) {
  gpt2::set_global_error(fmt, path ? path : "(null)");
  return code;
}

// element counts of the 16 parameter tensors (section 1.22)
size_t count_params(int maxT, int V, int L, int C) {
  const size_t c = C, l = L;
  const size_t n[16] = {(size_t)V * c, (size_t)maxT * c, l * c, l * c, l * 3 * c * c, l * 3 * c,
                        l * c * c, l * c, l * c, l * c, l * 4 * c * c, l * 4 * c,
                        l * c * 4 * c, l * c, c, c};
  size_t total = 0;
  for (size_t x : n) total += x;
  return total;
}

struct Header {
  int maxT, V, L, NH, C;
  size_t nparams;
};

// reads and checks the header; on success the file is positioned at the parameters
int read_header(FILE* f, const char* path, Header* h) {
  int32_t hdr[kHeaderInts];
  if (fread(hdr, sizeof(int32_t), kHeaderInts, f) != (size_t)kHeaderInts)
    return io_fail(GPT2_ERR_IO, "checkpoint %s: shorter than its 256-int header", path);
  if (hdr[0] != kMagic) return io_fail(GPT2_ERR_IO, "checkpoint %s: bad magic number", path);
  if (hdr[1] != kVersion) return io_fail(GPT2_ERR_IO, "checkpoint %s: unsupported version", path);
  h->maxT = hdr[2];
  h->V = hdr[3];
  h->L = hdr[4];
  h->NH = hdr[5];
  h->C = hdr[6];
  if (h->maxT < 1 || h->V < 1 || h->L < 1 || h->NH < 1 || h->C < 1)
    return io_fail(GPT2_ERR_IO, "checkpoint %s: non-positive size in the header", path);
  h->nparams = count_params(h->maxT, h->V, h->L, h->C);
  if (fseek(f, 0, SEEK_END) != 0) return io_fail(GPT2_ERR_IO, "checkpoint %s: seek failed", path);
  const long size = ftell(f);
  const long want = (long)(kHeaderInts * sizeof(int32_t) + h->nparams * sizeof(float));
  if (size != want)
    return io_fail(GPT2_ERR_IO, "checkpoint %s: file size does not match its header", path);
  if (fseek(f, kHeaderInts * sizeof(int32_t), SEEK_SET) != 0)
    return io_fail(GPT2_ERR_IO, "checkpoint %s: seek failed", path);
  return GPT2_OK;
}

}  // namespace

// ----- checkpoints ----------------------------------------------------------------------

extern "C" int gpt2_checkpoint_info(const char* path, int* maxT, int* V, int* L, int* NH, int* C,
                                    size_t* num_params) {
  if (!path) return io_fail(GPT2_ERR_ARG, "gpt2_checkpoint_info: NULL path%s", "");
  FILE* f = fopen(path, "rb");
  if (!f) return io_fail(GPT2_ERR_IO, "checkpoint %s: cannot open", path);
  Header h;
  const int rc = read_header(f, path, &h);
  fclose(f);
  if (rc) return rc;
  if (maxT) *maxT = h.maxT;
  if (V) *V = h.V;
  if (L) *L = h.L;
  if (NH) *NH = h.NH;
  if (C) *C = h.C;
  if (num_params) *num_params = h.nparams;
  return GPT2_OK;
}

extern "C" int gpt2_checkpoint_read(const char* path, float* params, size_t n) {
  if (!path || !params) return io_fail(GPT2_ERR_ARG, "gpt2_checkpoint_read: NULL argument%s", "");
  FILE* f = fopen(path, "rb");
  if (!f) return io_fail(GPT2_ERR_IO, "checkpoint %s: cannot open", path);
  Header h;
  int rc = read_header(f, path, &h);
  if (!rc && n != h.nparams) rc = io_fail(GPT2_ERR_ARG, "checkpoint %s: buffer size differs "
                                          "from the checkpoint's parameter count", path);
  if (!rc && fread(params, sizeof(float), n, f) != n)
    rc = io_fail(GPT2_ERR_IO, "checkpoint %s: read failed", path);
  fclose(f);
  return rc;
}

extern "C" int gpt2_checkpoint_write(const char* path, int maxT, int V, int L, int NH, int C,
                                     const float* params) {
  if (!path || !params || maxT < 1 || V < 1 || L < 1 || NH < 1 || C < 1)
    return io_fail(GPT2_ERR_ARG, "gpt2_checkpoint_write: bad argument for %s", path);
  int32_t hdr[kHeaderInts];
  memset(hdr, 0, sizeof(hdr));
  hdr[0] = kMagic;
  hdr[1] = kVersion;
  hdr[2] = maxT;
  hdr[3] = V;
  hdr[4] = L;
  hdr[5] = NH;
  hdr[6] = C;
  const size_t n = count_params(maxT, V, L, C);
  FILE* f = fopen(path, "wb");
  if (!f) return io_fail(GPT2_ERR_IO, "checkpoint %s: cannot create", path);
  bool ok = fwrite(hdr, sizeof(int32_t), kHeaderInts, f) == (size_t)kHeaderInts &&
            fwrite(params, sizeof(float), n, f) == n;
  ok = (fclose(f) == 0) && ok;
  return ok ? GPT2_OK : io_fail(GPT2_ERR_IO, "checkpoint %s: write failed", path);
}

extern "C" int gpt2_build_from_checkpoint(gpt2_model** out, const char* path, int dtype,
                                          int maxB, int maxTseq, void* stream) {
  if (!out) return io_fail(GPT2_ERR_ARG, "gpt2_build_from_checkpoint: NULL handle%s", "");
  *out = nullptr;
  int maxT, V, L, NH, C;
  size_t n;
  int rc = gpt2_checkpoint_info(path, &maxT, &V, &L, &NH, &C, &n);
  if (rc) return rc;
  std::vector<float> host(n);
  rc = gpt2_checkpoint_read(path, host.data(), n);
  if (rc) return rc;
  gpt2_model* md = nullptr;
  rc = gpt2_build_ex(&md, L, C, NH, V, maxT, dtype, maxB, maxTseq, stream);
  if (rc) return rc;
  rc = gpt2_set_params(md, host.data(), 0);
  if (!rc) rc = gpt2_synchronize(md);
  if (rc) {
    gpt2_free(md);
    return rc;
  }
  *out = md;
  return GPT2_OK;
}

extern "C" int gpt2_save_checkpoint(gpt2_model* model, const char* path) {
  if (!model || !path) return io_fail(GPT2_ERR_ARG, "gpt2_save_checkpoint: NULL argument%s", "");
  int cfg[5];
  int rc = gpt2_get_config(model, cfg);
  if (rc) return rc;
  std::vector<float> host(gpt2_num_params(model));
  rc = gpt2_get_params(model, host.data(), 0);
  if (rc) return rc;
  return gpt2_checkpoint_write(path, cfg[4], cfg[3], cfg[0], cfg[2], cfg[1], host.data());
}

// ----- token files (DataLoader) -----------------------------------------------------------

struct gpt2_dataloader {
  int B = 0, T = 0;
  FILE* file = nullptr;
  long file_size = 0;
  long position = 0;
  std::vector<int32_t> window;  // B*T + 1 tokens
};

extern "C" int gpt2_dataloader_init(gpt2_dataloader** out, const char* path, int B, int T) {
  if (!out || !path || B < 1 || T < 1)
    return io_fail(GPT2_ERR_ARG, "gpt2_dataloader_init: bad argument for %s", path);
  *out = nullptr;
  FILE* f = fopen(path, "rb");
  if (!f) return io_fail(GPT2_ERR_IO, "token file %s: cannot open", path);
  if (fseek(f, 0, SEEK_END) != 0) {
    fclose(f);
    return io_fail(GPT2_ERR_IO, "token file %s: seek failed", path);
  }
  const long size = ftell(f);
  const long need = ((long)B * T + 1) * (long)sizeof(int32_t);
  if (size < need) {
    fclose(f);
    return io_fail(GPT2_ERR_ARG, "token file %s: smaller than one batch of B*T+1 tokens", path);
  }
  auto* dl = new gpt2_dataloader;
  dl->B = B;
  dl->T = T;
  dl->file = f;
  dl->file_size = size;
  dl->position = 0;
  dl->window.resize((size_t)B * T + 1);
  *out = dl;
  return GPT2_OK;
}

extern "C" int gpt2_dataloader_num_batches(const gpt2_dataloader* dl) {
  if (!dl) return 0;
  return (int)(dl->file_size / ((long)dl->B * dl->T * (long)sizeof(int32_t)));
}

extern "C" int gpt2_dataloader_reset(gpt2_dataloader* dl) {
  if (!dl) return io_fail(GPT2_ERR_ARG, "gpt2_dataloader_reset: NULL loader%s", "");
  dl->position = 0;
  return GPT2_OK;
}

extern "C" int gpt2_dataloader_next_batch(gpt2_dataloader* dl, int32_t* inputs, int32_t* targets,
                                          int dst_is_device, void* stream) {
  if (!dl || !inputs || !targets)
    return io_fail(GPT2_ERR_ARG, "gpt2_dataloader_next_batch: NULL argument%s", "");
  const long bt = (long)dl->B * dl->T;
  const long span = (bt + 1) * (long)sizeof(int32_t);
  if (dl->position + span > dl->file_size) dl->position = 0;
  if (fseek(dl->file, dl->position, SEEK_SET) != 0 ||
      fread(dl->window.data(), sizeof(int32_t), bt + 1, dl->file) != (size_t)(bt + 1))
    return io_fail(GPT2_ERR_IO, "token file read failed%s", "");
  dl->position += bt * (long)sizeof(int32_t);
  if (!dst_is_device) {
    memcpy(inputs, dl->window.data(), bt * sizeof(int32_t));
    memcpy(targets, dl->window.data() + 1, bt * sizeof(int32_t));
    return GPT2_OK;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  GPT2_HIP_OK(hipMemcpyAsync(inputs, dl->window.data(), bt * sizeof(int32_t),
                             hipMemcpyHostToDevice, s));
  GPT2_HIP_OK(hipMemcpyAsync(targets, dl->window.data() + 1, bt * sizeof(int32_t),
                             hipMemcpyHostToDevice, s));
  // the window is refilled by the next call: wait until the copies have read it
  GPT2_HIP_OK(hipStreamSynchronize(s));
  return GPT2_OK;
}

extern "C" void gpt2_dataloader_free(gpt2_dataloader* dl) {
  if (!dl) return;
  if (dl->file) fclose(dl->file);
  delete dl;
}

// ----- random numbers (sections 1.33, 1.34) ----------------------------------------------

// xorshift* (Marsaglia's xorshift with shifts 12, 25, 27, then a multiplication by
// 0x2545F4914F6CDD1D, keeping the upper 32 bits of the product)
extern "C" uint32_t gpt2_random_u32(uint64_t* state) {
  uint64_t x = *state;
  x ^= x >> 12;
  x ^= x << 25;
  x ^= x >> 27;
  *state = x;
  return (uint32_t)((x * 0x2545F4914F6CDD1DULL) >> 32);
}

// the upper 24 bits of the next draw over 2^24: a float in [0, 1)
extern "C" float gpt2_random_f32(uint64_t* state) {
  return (float)(gpt2_random_u32(state) >> 8) / 16777216.0f;
}
