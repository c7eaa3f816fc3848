// Status codes shared by the host metadata layer and the C-ABI (values equal
// the mkv_status enum of include/mkv.h).
#pragma once

#define MKV_S_OK 0
#define MKV_S_EINVAL (-1)
#define MKV_S_ENOMEM (-2)
#define MKV_S_ESTATE (-3)
#define MKV_S_ERANGE (-4)
#define MKV_S_EHIP (-5)
