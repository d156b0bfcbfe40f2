// Copy of a built segment table to the device on the caller's stream.

#include "device.h"

extern "C" int asv_table_upload(const void* blob, size_t bytes, void* dev_blob, void* stream) {
  if (blob == nullptr || dev_blob == nullptr || !asv::aligned16(dev_blob)) return ASV_E_ARG;
  if (bytes == 0) return ASV_OK;
  const hipError_t e = hipMemcpyAsync(dev_blob, blob, bytes, hipMemcpyHostToDevice,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ASV_OK : ASV_E_HIP;
}
