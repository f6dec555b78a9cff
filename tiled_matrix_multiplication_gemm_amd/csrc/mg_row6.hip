// Kernels of table row 6 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW(6, Cfg6, Fast6)
